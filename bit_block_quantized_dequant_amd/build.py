"""Build libq4gemv.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m bit_block_quantized_dequant_amd.build [-v]

The library is built into this package directory so that it travels with the
source tree; it is compiled for gfx950 only.  Packed-fp32 instructions are
disabled (-packed-fp32-ops): the kernels use scalar fp32 and mixed-precision
FMAs only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4gemv.so")
SOURCES = [os.path.join(CSRC, "q4gemv.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("q4_device.h", "q4_kernels.h", "q4_mfma.h",
                                                  "q4_router.h")] + [
    os.path.join(ROOT, "include", "q4gemv.h")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp] + list(extra) + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
