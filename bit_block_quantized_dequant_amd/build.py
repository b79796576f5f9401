"""Build libq4gemv.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m bit_block_quantized_dequant_amd.build [-v]

The library is built into this package directory so that it travels with the
source tree; it is compiled for gfx950 only.  Each csrc/*.hip translation
unit (the entry points of a group of calls and the kernels they instantiate)
compiles in parallel, and they are linked into one shared library.
Packed-fp32 instructions are disabled (-packed-fp32-ops): the kernels use
scalar fp32 and mixed-precision FMAs only.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4gemv.so")
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
DEPS = SOURCES + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")) + [
    os.path.join(ROOT, "include", "q4gemv.h")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd, verbose):
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


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every translation unit (in parallel) and link libq4gemv.so."""
    tag = "%d" % os.getpid()
    objdir = os.path.join(ROOT, "_build", "q4gemv_" + tag)
    os.makedirs(objdir, exist_ok=True)
    flags = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + list(extra)
    objs = [os.path.join(objdir, os.path.basename(src)[:-4] + ".o") for src in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [hipcc()] + flags + ["-c", src, "-o", obj], verbose)
                for src, obj in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp" + tag
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    os.rmdir(objdir)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
