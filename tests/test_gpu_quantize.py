"""GPU parity of kvq_quantize_pack: the packed bytes (codes, fp16 scale/zero, hybrid flags)
must equal the CPU oracle's bit for bit, on several blocks with assorted value shapes,
on strided sources, at a block offset, and on the full-size workloads."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

FORMATS = [(4, False), (3, False), (2, False), (2, True), (3, True), (4, True)]


def _special_rows(rng, rows, T):
    """Rows mixing ordinary values with groups that hit the quantizer's corner cases."""
    x = S.random_groups(rng, rows * T * 4, "t5").reshape(rows, T, 128)
    kinds = ["normal", "wide", "tiny", "offset", "few_levels", "ternary"]
    for i, kind in enumerate(kinds):
        x[i % rows, 7 * i:7 * i + 5] = S.random_groups(rng, 5 * 4, kind).reshape(5, 128)
    x[0, 100, :32] = np.float16(2.5)                 # constant group
    x[0, 101, 32:64] = np.float16(-0.0)              # all -0.0
    x[1, 102, 64:96] = np.float16(0.0)
    x[1, 102, 64] = np.float16(2.0 ** -24)           # scale underflows to 0
    x[1, 103, :32] = np.array([0.0, 22 * 2 ** -24] + [7 * 2 ** -24] * 30, np.float32).astype(np.float16)
    x[0, 104, :32] = np.float16(0.0)
    x[0, 104, :3] = np.array([-40000.0, 40000.0, 0.0], np.float32).astype(np.float16)
    x[1, 105, 96:] = np.float16(65504.0)
    x[1, 105, 96] = np.float16(-65504.0)             # full fp16 range in one group
    return x


@pytest.mark.parametrize("bits,hybrid", FORMATS)
def test_quantize_bit_exact_small(oracle_mod, bits, hybrid):
    from gpu_common import gpu_quantize
    O = oracle_mod
    rng = np.random.default_rng(1000 + bits + 10 * hybrid)
    rows, T = 3, 384
    src = _special_rows(rng, rows, T)
    fmt = K.Format(bits, 128, hybrid)
    print(f"[quantize small] bits={bits} hybrid={hybrid} rows={rows} T={T}", flush=True)
    got = gpu_quantize(fmt, src).cpu().numpy()
    ref = O.quantize_pack(O.Format(bits, 128, hybrid), src)
    assert got.shape == ref.shape
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def _boundary_rows(rng, bits, rows, T):
    """Groups whose values sit at, and a few fp16 steps around, the half-integer points
    zero + (k + 1/2) * scale where the code changes, for the scale the group's own min and
    max give; half of the groups have a zero point so small that x - zero keeps bits far
    below x's own precision (quotients close to, but not on, a half-integer)."""
    N = (1 << bits) - 1
    G = rows * T * 4
    mag = 2.0 ** rng.uniform(-12, 8, G)
    z = np.where(rng.random(G) < 0.5, -mag * rng.uniform(0.0, 1.0, G),
                 rng.choice([-1.0, 1.0], G) * 2.0 ** rng.uniform(-24, -14, G))
    z16 = z.astype(np.float16)
    mx16 = (z16.astype(np.float64) + mag).astype(np.float16)
    # the scale the quantizer derives from this min and max (fp32 arithmetic, then fp16)
    s = ((mx16.astype(np.float32) - z16.astype(np.float32)) / np.float32(N)).astype(np.float16)
    k = rng.integers(0, N, (G, 30))
    tie = z16.astype(np.float64)[:, None] + (k + 0.5) * s.astype(np.float64)[:, None]
    x = tie.astype(np.float16)
    for _ in range(4):                               # up to 4 fp16 steps either way
        step = rng.integers(-1, 2, x.shape)
        x = np.where(step > 0, np.nextafter(x, np.float16(np.inf)),
                     np.where(step < 0, np.nextafter(x, np.float16(-np.inf)), x))
    lo, hi = np.minimum(z16, mx16), np.maximum(z16, mx16)
    x = np.clip(x, lo[:, None], hi[:, None])
    grp = np.concatenate([z16[:, None], mx16[:, None], x], axis=1)
    perm = rng.permuted(np.tile(np.arange(32), (G, 1)), axis=1)
    grp = np.take_along_axis(grp, perm, axis=1)
    return np.ascontiguousarray(grp.reshape(rows, T, 128))


@pytest.mark.parametrize("bits,hybrid", FORMATS)
def test_quantize_rounding_boundaries(oracle_mod, bits, hybrid):
    """Codes of values at and next to the points where rounding changes (the kernel rounds a
    reciprocal-based quotient and redoes the ones near such a point with the correctly
    rounded division): bytes equal to the oracle's."""
    from gpu_common import gpu_quantize
    O = oracle_mod
    rng = np.random.default_rng(1200 + bits + 10 * hybrid)
    src = _boundary_rows(rng, bits, 4, 256)
    fmt = K.Format(bits, 128, hybrid)
    print(f"[quantize boundaries] bits={bits} hybrid={hybrid}", flush=True)
    got = gpu_quantize(fmt, src).cpu().numpy()
    ref = O.quantize_pack(O.Format(bits, 128, hybrid), src)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def _random_quant_cases(n, seed=77):
    rng = np.random.default_rng(seed)
    kinds = ["normal", "t5", "wide", "tiny", "offset", "few_levels", "ternary"]
    return [(i, int(rng.choice([2, 3, 4])), bool(rng.random() < 0.4),
             str(rng.choice(kinds)), int(rng.integers(1, 6)), 128 * int(rng.integers(1, 5)),
             int(rng.integers(0, 3)), int(rng.integers(0, 3))) for i in range(n)]


@pytest.mark.parametrize("case", _random_quant_cases(12), ids=lambda c: f"r{c[0]}_{c[3]}")
def test_quantize_random_shapes(oracle_mod, case):
    """Seeded random formats, value shapes, row counts, token counts, padded token strides and
    block offsets: packed bytes equal to the oracle's."""
    from gpu_common import DEV, dev
    O = oracle_mod
    i, bits, hybrid, kind, rows, T, pad, fb = case
    rng = np.random.default_rng(1300 + i)
    tok_stride = 128 + 8 * pad                        # padded token rows (16-byte multiples)
    x = S.random_groups(rng, rows * T * 4, kind).reshape(rows, T, 128)
    src = np.zeros((rows, T, tok_stride), np.float16)
    src[:, :, :128] = x
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    bb = fmt.block_bytes
    cap = fb + T // 128
    print(f"[quantize random] case={case}", flush=True)
    dst = torch.zeros((rows, cap * bb), dtype=torch.uint8, device=DEV)
    K.kvq_quantize_pack(fmt, dev(src), rows, T, T * tok_stride, tok_stride, dst, cap * bb, fb)
    ref = O.quantize_pack(ofmt, np.ascontiguousarray(x), n_blocks_capacity=cap, first_block=fb)
    got = dst.cpu().numpy()
    bad = np.flatnonzero(got[:, fb * bb:] != ref[:, fb * bb:])
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
    assert not got[:, :fb * bb].any(), "bytes before the first block were written"


@pytest.mark.parametrize("bits,hybrid", [(4, False), (2, True), (3, False)])
def test_quantize_strided_source_and_block_offset(oracle_mod, bits, hybrid):
    """Quantize tokens [128, 384) of a [B][H][L][d] tensor into blocks 2.. of a wider
    cache: the source row stride is L*d and tokens start mid-tensor."""
    from gpu_common import DEV, dev
    O = oracle_mod
    rng = np.random.default_rng(1100 + bits)
    B, H, L = 2, 3, 512
    x = S.random_groups(rng, B * H * L * 4, "normal").reshape(B, H, L, 128)
    fmt = K.Format(bits, 128, hybrid)
    bb = fmt.block_bytes
    cap = 6
    dst = torch.full((B * H, cap * bb), 0xAB, dtype=torch.uint8, device=DEV)
    xt = dev(x)
    print(f"[quantize strided] bits={bits} hybrid={hybrid}", flush=True)
    first_tok = xt.data_ptr() + 128 * 128 * 2          # token 128 of row 0 (64-B aligned)
    K.kvq_quantize_pack(fmt, first_tok, B * H, 256, L * 128, 128, dst, cap * bb, 2)
    got = dst.cpu().numpy()
    ref = np.full((B * H, cap * bb), 0xAB, np.uint8)
    O.quantize_pack(O.Format(bits, 128, hybrid), np.ascontiguousarray(
        x.reshape(B * H, L, 128)[:, 128:384]), first_block=2, dst=ref)
    assert np.array_equal(got, ref)


def test_quantize_deterministic():
    from gpu_common import gpu_quantize
    rng = np.random.default_rng(1200)
    src = S.random_groups(rng, 16 * 512 * 4, "t5").reshape(16, 512, 128)
    fmt = K.Format(2, 128, True)
    print("[quantize determinism]", flush=True)
    a = gpu_quantize(fmt, src)
    b = gpu_quantize(fmt, src)
    assert torch.equal(a, b)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "batch8_2bit_hybrid", "long_128k_3bit",
                                  "mha_b64_append"])
def test_quantize_full_workload_bit_exact(oracle_mod, name):
    from gpu_common import gpu_quantize
    O = oracle_mod
    wl = S.WORKLOADS[name]
    print(f"[quantize full] {name}: generating inputs", flush=True)
    x = S.make_inputs(wl)
    kp_src, vp_src = x.packed_src()
    fmt = K.Format(wl.bits, 128, wl.hybrid)
    ofmt = O.Format(wl.bits, 128, wl.hybrid)
    rows = wl.B * wl.Hkv
    flags_sym = 0
    for name_kv, src in (("K", kp_src), ("V", vp_src)):
        src = np.ascontiguousarray(src.reshape(rows, wl.n_packed, 128))
        print(f"[quantize full] {name}: {name_kv} rows={rows} T={wl.n_packed}", flush=True)
        got = gpu_quantize(fmt, src).cpu().numpy()
        ref = O.quantize_pack(ofmt, src)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, f"{name} {name_kv}: {bad.size} bytes differ, first at {bad[:8]}"
        if wl.hybrid:
            bb = fmt.block_bytes
            fl = ref.reshape(rows, -1, bb)[:, :, fmt.flag_offset:fmt.flag_offset + 64]
            flags_sym += int(np.unpackbits(fl).size - np.unpackbits(fl).sum())
        del got, ref
    if wl.hybrid:
        total = 2 * rows * wl.n_packed * 4
        print(f"[quantize full] {name}: symmetric-mode groups {flags_sym / total:.4%}", flush=True)
