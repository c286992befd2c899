"""Build the HIP library libllmint8.so for gfx950 with hipcc, in-tree.

Flags that matter for results:
  * -fhip-fp32-correctly-rounded-divide-sqrt: the int8 quantization takes
    round(127*x/a) through r = 127/a and x*r where that is provably the same
    rounding, and from one IEEE-correct fp32 division otherwise; both
    divisions must be correctly rounded;
  * no fast-math;
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU
    instructions are generated.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libllmint8.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "decode.hip", "ceiling.hip"]
ARCH = os.environ.get("LLMINT8_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False):
    """Compile every HIP source into libllmint8.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the gfx950 feature flag and says so once
    # per source; keep every other line of the compiler output
    msgs = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if msgs:
        print("\n".join(msgs), flush=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (exit %d)" % r.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
