"""The build's numeric contract, checked on the CPU: the library's compile flags keep fp16
and fp32 denormals (the decode's matrix-core operands are fp16 subnormals), and a kernel
compiled with exactly those flags carries the preserving denormal modes in its
descriptor."""
import os
import re
import shutil
import subprocess

import pytest

from bit_kv_cache_pack_amd import build as B

FLUSHING = ("-ffast-math", "-Ofast", "-funsafe-math-optimizations", "-ffinite-math-only",
            "-fgpu-flush-denormals-to-zero", "-fcuda-flush-denormals-to-zero")


def test_flags_preserve_denormals():
    flags = B.compile_flags()
    assert "-fdenormal-fp-math=ieee" in flags
    for f in flags:
        assert f not in FLUSHING, f
        m = re.match(r"-fdenormal-fp-math(-f32)?=(.*)", f)
        if m:
            assert m.group(2) == "ieee", f


def test_compiled_kernel_keeps_denormals(tmp_path):
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    src = tmp_path / "probe.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   "__global__ void probe(const _Float16 *a, float *o)\n"
                   "{ o[threadIdx.x] = (float)a[threadIdx.x] * 2.0f; }\n")
    asm = tmp_path / "probe.s"
    r = subprocess.run([hipcc, *B.compile_flags(), "--cuda-device-only", "-S", "-o", str(asm),
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    txt = asm.read_text()
    m16 = re.findall(r"\.amdhsa_float_denorm_mode_16_64\s+(\d+)", txt)
    m32 = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", txt)
    assert m16 and set(m16) == {"3"}, m16      # 3: fp16/fp64 denormals in and out
    assert m32 and set(m32) == {"3"}, m32
