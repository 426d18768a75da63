"""Build libkvq.so (HIP for gfx950) in-tree with hipcc.

    python -m bit_kv_cache_pack_amd.build        # or build() from Python

Flags: -O3 for gfx950 only; packed-FP32 instructions disabled; fp32 division and square
root correctly rounded (the quantizer's codes must equal the CPU definition bit for bit).

Denormals are a build contract: every kernel must run with fp16 (and fp32) denormals
preserved, not flushed. The decode feeds the K and V codes to the matrix cores as fp16
subnormals (a code in the low mantissa bits of a half with a zero exponent field is
exactly code * 2^-24); with fp16 denormals flushed every such operand would read as 0.
`-fdenormal-fp-math=ieee` states the mode explicitly (the kernel descriptors then carry
float_denorm_mode 3 for fp16/fp64 and fp32), and no fast-math or flush option may be
added: tests/test_build_contract.py checks both, on the flags and on a kernel compiled
with them.
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
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-fdenormal-fp-math=ieee",
            "-Wall", "-Wno-unused-function",
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


# The host side of the library (the C ABI's argument checks) with GPU launches replaced by
# launchers that launch nothing, compiled by the host compiler under AddressSanitizer and
# UndefinedBehaviorSanitizer. Load it with the sanitizer runtime preloaded
# (LD_PRELOAD=$(gcc -print-file-name=libasan.so)) and point KVQ_LIB_PATH at it.
HOST_CHECKED_SOURCES = ["kvq_api.cpp", "host_only_launchers.cpp"]


def build_host_checked(out: str, verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(rocm, "include"), "-I", INCLUDE,
           "-I", CSRC, "-o", out, *[os.path.join(CSRC, s) for s in HOST_CHECKED_SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
