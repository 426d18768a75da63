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


# ---- direct-to-LDS loads: the LDS base (M0) must be one wave-uniform value -------------
# A direct-to-LDS buffer load writes lane i's bytes at M0 + size * i. When the compiler
# merges two such calls with different LDS pointers (one under a lane condition, one not)
# into one call on a per-lane pointer, it sets M0 from v_readfirstlane of that pointer:
# every lane then writes relative to lane 0's base, silently overwriting the wrong part of
# LDS. This was seen with a reordered 3-bit tile load; the check keeps it from coming back.

_WRITES = re.compile(r"^\s*(?:s_|v_readfirstlane)\S*\s+(s\d+|s\[(\d+):(\d+)\])\s*,")


def _sgpr_range(tok, lo, hi):
    if lo is not None:
        return range(int(lo), int(hi) + 1)
    return range(int(tok[1:]), int(tok[1:]) + 1)


def _m0_from_readfirstlane(asm_text):
    bad = []
    lines = asm_text.splitlines()
    for k, line in enumerate(lines):
        m = re.match(r"^\s*s_\w+\s+m0\s*,\s*(s\d+)", line)
        if not m:
            continue
        reg = int(m.group(1)[1:])
        for j in range(k - 1, max(k - 400, -1), -1):
            prev = lines[j]
            if re.match(r"^\S.*:\s*(;.*)?$", prev) and not prev.startswith(("\t", " ")):
                if re.match(r"^[._A-Za-z0-9]+:", prev) and not prev.startswith(".LBB"):
                    break                                     # start of another function
            w = _WRITES.match(prev)
            if w and reg in _sgpr_range(w.group(1), w.group(2), w.group(3)):
                if prev.strip().startswith("v_readfirstlane"):
                    bad.append((k, prev.strip(), line.strip()))
                break
    return bad


def test_scanner_flags_m0_from_readfirstlane():
    asm = ("_Z1kv:\n\tv_readfirstlane_b32 s10, v4\n\ts_mov_b32 s42, s38\n"
           "\ts_mov_b32 m0, s10\n\tbuffer_load_dwordx4 v2, s[40:43], 0 offen lds\n"
           "\ts_add_i32 s11, s33, 0x400\n\ts_mov_b32 m0, s11\n")
    bad = _m0_from_readfirstlane(asm)
    assert len(bad) == 1 and "v_readfirstlane" in bad[0][1]


@pytest.mark.parametrize("src", ["decode_attn.hip", "decode_valu.hip"])
def test_lds_dma_base_is_uniform(tmp_path, src):
    """No M0 in the kernels that load tiles straight into LDS comes from v_readfirstlane."""
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    asm = tmp_path / (src + ".s")
    r = subprocess.run([hipcc, *B.compile_flags(), "--cuda-device-only", "-S", "-o", str(asm),
                        os.path.join(B.CSRC, src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad = _m0_from_readfirstlane(asm.read_text())
    assert not bad, bad[:3]
