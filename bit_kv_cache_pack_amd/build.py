"""Build libkvq.so (HIP for gfx950) in-tree with hipcc.

    python -m bit_kv_cache_pack_amd.build        # or build() from Python

Flags: -O3 for gfx950 only; packed-FP32 instructions disabled; fp32 division and square
root correctly rounded (the quantizer's codes must equal the CPU definition bit for bit).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_api.cpp", "quant_pack.hip", "decode_attn.hip", "decode_valu.hip", "combine.hip",
           "keynorm.hip", "paged.hip", "quant_outer.hip", "stream_read.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def compile_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall", "-Wno-unused-function",
            # MFMA accumulators in ordinary VGPRs: the online-softmax rescale multiplies
            # them every tile, which would otherwise copy them out of and back into AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), *extra, "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name and says so; that is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
