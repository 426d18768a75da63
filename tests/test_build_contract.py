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


def _asm_statements(text):
    """(template, output operands) of every GCC-style asm statement in a source text (colons
    inside string literals do not separate operand lists)."""
    out = []
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(", text):
        i, depth, in_str, sections = m.end(), 1, False, [""]
        while i < len(text):
            c = text[i]
            if in_str:
                if c == "\\":
                    sections[-1] += text[i:i + 2]
                    i += 2
                    continue
                if c == '"':
                    in_str = False
                sections[-1] += c
            elif c == '"':
                in_str = True
                sections[-1] += c
            elif c == "(":
                depth += 1
                sections[-1] += c
            elif c == ")":
                depth -= 1
                if depth == 0:
                    break
                sections[-1] += c
            elif c == ":" and depth == 1:
                sections.append("")
            else:
                sections[-1] += c
            i += 1
        tmpl = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', sections[0]))
        out.append((tmpl, sections[1] if len(sections) > 1 else ""))
    return out


def test_no_inline_asm_vgpr_writes():
    """No kernel source writes a VGPR from an inline asm instruction. The compiler does not
    count inline asm as a VALU write when it inserts the wait states a matrix-core (MFMA)
    instruction needs after a VALU write of its operands (or before a VALU overwrite of an
    accumulator it is still reading), so such a write next to an MFMA can feed it a stale
    value. Empty templates (register-allocation barriers) and instructions with no VGPR
    output (waits, priorities) are allowed."""
    csrc = B.CSRC
    bad = []
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        text = open(os.path.join(csrc, name)).read()
        for tmpl, outputs in _asm_statements(text):
            if tmpl.strip() and re.search(r'"[=+&]*v"', outputs):
                bad.append(f"{name}: {tmpl.strip()}")
    assert not bad, bad
