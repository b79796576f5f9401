"""Plant plausible mistakes in copies of the CPU oracle and show that the pins
catch every one of them (the pins are only worth something if they do).

Each mutant is one textual edit of oracle/q4_oracle.c, compiled with gcc into
a temporary directory and bound with oracle.oracle.Oracle; the pins of
oracle_pins.py run in order until one fails.  Nothing here touches a GPU."""
import os
import subprocess
import tempfile

import pytest

import oracle_pins as P
from oracle.oracle import Oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q4_oracle.c")

MUTANTS = {
    "q4_0 offset 8 -> 7": ("(double)(hi - 8)", "(double)(hi - 7)"),
    "q4_0 low/high nibble swapped": ("int lo = qs[j] & 0x0F;", "int lo = qs[j] >> 4;"),
    "q4_0 high element j+16 -> j+8": ("out[j + 16] =", "out[j + 8] ="),
    "q4k min of sub-blocks 4-7 from S[j-4]": ("*m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);",
                                              "*m = (S[j + 4] >> 4) | ((S[j - 4] >> 6) << 4);"),
    "q4k scale of 4-7 without high bits": ("*sc = (S[j + 4] & 0x0F) | ((S[j - 4] >> 6) << 4);",
                                           "*sc = (S[j + 4] & 0x0F);"),
    "q4k 6-bit mask 63 -> 31": ("*sc = S[j] & 63;", "*sc = S[j] & 31;"),
    "q4k chunk of 64 -> consecutive nibbles": ("int q = (qs[32 * c + i] >> (4 * h)) & 0x0F;",
                                               "int q = (qs[t / 2] >> (4 * (t % 2))) & 0x0F;"),
    "q4k sub-block index from chunk": ("oracle_q4k_scale_min(S, t / 32, &sc, &m);",
                                       "oracle_q4k_scale_min(S, c + h, &sc, &m);"),
    "q4k min sign flipped": ("- dmin * (double)m);", "+ dmin * (double)m);"),
    "q4k d and dmin swapped": ("double d = f16_value(le16(sb));",
                               "double d = f16_value(le16(sb + 2));"),
    "f16 exponent bias off by one": ("expo - 25", "expo - 24"),
    "f16 subnormal scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "gemv drops first product": ("for (int64_t k = 0; k < j->K; ++k) {",
                                 "for (int64_t k = 1; k < j->K; ++k) {"),
    "gemv absdot without abs": ("aacc += fabs(p);", "aacc += p;"),
    "rmsnorm mean over K-1": ("ss / (double)K", "ss / (double)(K - 1)"),
    "rmsnorm drops gamma": ("(xm[k] * r) * gamma[k]", "(xm[k] * r)"),
    "rmsnorm drops eps": ("sqrtf(ms + eps)", "sqrtf(ms)"),
    "moe uses token 0 for every token": ("x + m * K, 1, N, K, g", "x, 1, N, K, g"),
    "moe gate/up matrices swapped": ("oracle_q4_0_gemv(wg + e * mat_bytes",
                                     "oracle_q4_0_gemv(wu + e * mat_bytes"),
    "checksum byte order": ("((uint32_t)r[b + 2] << 16)", "((uint32_t)r[b + 2] << 8)"),
    "silu sigmoid of +g": ("exp(-g[i])", "exp(g[i])"),
    "silu drops up": ("h[i] = s * u[i];", "h[i] = s;"),
    "top-k ties to the higher index": ("if (best < 0 || v > bv) {", "if (best < 0 || v >= bv) {"),
    "softmax without the max shift": ("return exp(v - lmax);", "return exp(v);"),
    "softmax tie at an infinite maximum as exp(nan)": ("if (v == lmax) return 1.0;", ""),
    "softmax zero denominator unguarded": ("den > 0.0 ? t / den : 0.0", "t / den"),
    "softmax max includes NaN as +inf": (
        "if (!isnan(l[e]) && (isnan(lmax) || l[e] > lmax)) lmax = l[e];",
        "if (isnan(l[e]) || isnan(lmax) || l[e] > lmax) lmax = isnan(l[e]) ? INFINITY : l[e];"),
    "rmsnorm gamma index reversed": ("(xm[k] * r) * gamma[k]", "(xm[k] * r) * gamma[K - 1 - k]"),
    "normalize flag ignored": ("if (normalize) {", "if (0) {"),
    "router logits of token 0 only": ("oracle_q4_0_gemv(w, x, M, E, K, l, a, 1);",
                                      "oracle_q4_0_gemv(w, x, 1, E, K, l, a, 1);"),
    "q4k tail rows of floor(K/256) super-blocks": (
        "return (K + Q4K_SB_ELEMS - 1) / Q4K_SB_ELEMS;", "return K / Q4K_SB_ELEMS;"),
    "q4k tail drops the last sub-block": (
        "int64_t cnt = K - k0 < Q4K_SB_ELEMS ? K - k0 : Q4K_SB_ELEMS;",
        "int64_t cnt = K - k0 < Q4K_SB_ELEMS ? K - k0 - 32 : Q4K_SB_ELEMS;"),
    "q4k gemv row stride of whole super-blocks": (
        ": q4k_row_superblocks(j->K) * Q4K_SB_BYTES;", ": (j->K / Q4K_SB_ELEMS) * Q4K_SB_BYTES;"),
    "down uses the token's row for every slot": (
        "h + p * K, 1, N, K, yp", "h + (p / top_k) * K, 1, N, K, yp"),
    "down ignores the expert id": ("oracle_q4_0_gemv(wd + e * mat_bytes", "oracle_q4_0_gemv(wd"),
    "down invalid id not NaN": ("yp[r] = NAN;", "yp[r] = 0.0;"),
    "soa offset 8 -> 0": ("(float)(d * (double)(v - 8))", "(float)(d * (double)v)"),
    "soa high nibble from the next byte": ("(q[j - 16] >> 4)", "(q[j - 15 < 16 ? j - 15 : 15] >> 4)"),
    "soa scale of the row's first block": ("le16(scales + 2 * (n * nb + b))",
                                           "le16(scales + 2 * (n * nb))"),
    "soa repack takes the scale from the nibbles": (
        "memcpy(scales + 2 * i, w + Q4_0_BLOCK_BYTES * i, 2);",
        "memcpy(scales + 2 * i, w + Q4_0_BLOCK_BYTES * i + 2, 2);"),
    "silu without g": ("double s = g[i] / (1.0 + exp(-g[i]));",
                       "double s = 1.0 / (1.0 + exp(-g[i]));"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(source, name):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, "mutation site not found: %r" % old
    mutated = source.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "m.c")
        so = os.path.join(td, "libm.so")
        with open(c, "w") as f:
            f.write(mutated)
        subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                        "-pthread", "-o", so, c, "-lm"], check=True)
        o = Oracle(so)
        caught = None
        for pin in P.ALL_PINS:
            try:
                pin(o)
            except AssertionError:
                caught = pin.__name__
                break
        assert caught is not None, "no pin caught mutant %r" % name
