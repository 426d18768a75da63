"""Pins of the oracle's outer-dimension (KIVI-style) grouping (InnerQ page sec. 1 and
sec. 4.1 compare against it): groups of 32 consecutive tokens of one channel.

- a 128x128 block grouped along tokens is the (pinned) inner quantizer applied to the
  transposed block: same scale, zero and codes group for group, read back by an
  independent Python reader of the bytes;
- a hand example with a closed form;
- attention over exact-grid blocks (every group on a 1/16 grid, so dequantization is
  exact) equals attention over the same fp16 values held in the fp16 window;
- the split partials merge to the one-pass result.
"""
import numpy as np
import pytest

import synth_inputs as S

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _code(block, bits, t, c, d=128):
    gb = 4 * bits
    w = int.from_bytes(block[t * (d // 32) * gb + (c // 32) * gb: t * (d // 32) * gb + (c // 32 + 1) * gb].tobytes(), "little")
    return (w >> (bits * (c % 32))) & ((1 << bits) - 1)


def _sz(block, off):
    return tuple(int(v) for v in block[off:off + 4].view(np.uint16))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_outer_block_is_inner_quantizer_on_the_transpose(oracle_mod, bits):
    O = oracle_mod
    rng = np.random.default_rng(bits)
    fmt = O.Format(bits, 128, False)
    rows = 2
    x = _f16(rng.standard_normal((rows, 256, 128)) * rng.uniform(0.05, 20, (rows, 1, 128)))
    x[0, :32, 5] = 3.0                                         # a constant group
    outer = O.quantize_pack_outer(fmt, x)
    bb, szo = fmt.block_bytes, fmt.sz_offset
    for r in range(rows):
        for blk in range(2):
            xt = np.ascontiguousarray(x[r, blk * 128:(blk + 1) * 128].T)     # [c][t]
            inner = O.quantize_pack(fmt, xt[None])[0]
            ob = outer[r, blk * bb:(blk + 1) * bb]
            for tg in range(4):
                for c in range(0, 128, 7):
                    # outer group (tg, c) == inner group (token c, group tg) of the transpose
                    assert _sz(ob, szo + (tg * 128 + c) * 4) == _sz(inner, szo + (c * 4 + tg) * 4)
                    for i in range(32):
                        assert _code(ob, bits, 32 * tg + i, c) == _code(inner, bits, c, 32 * tg + i)


def test_outer_hand_example(oracle_mod):
    O = oracle_mod
    fmt = O.Format(4, 128, False)
    x = np.zeros((1, 128, 128), np.float16)
    x[0, 32:64, 9] = np.arange(32) % 16          # tokens 32..63 of channel 9: 0..15 twice
    x[0, 0:32, 100] = -2.0                        # constant group
    x[0, 0, 100] = 13.0
    b = O.quantize_pack_outer(fmt, x)[0]
    s, z = _sz(b, fmt.sz_offset + (1 * 128 + 9) * 4)
    assert np.uint16(s).view(np.float16) == 1.0 and np.uint16(z).view(np.float16) == 0.0
    assert [_code(b, 4, 32 + i, 9) for i in range(32)] == [i % 16 for i in range(32)]
    s, z = _sz(b, fmt.sz_offset + (0 * 128 + 100) * 4)
    assert np.uint16(s).view(np.float16) == 1.0 and np.uint16(z).view(np.float16) == -2.0
    assert _code(b, 4, 0, 100) == 15 and _code(b, 4, 1, 100) == 0
    # an all-zero group: scale 0, codes 0
    assert _sz(b, fmt.sz_offset + (3 * 128 + 50) * 4) == (0, 0)


def _grid_block(rng, rows, T, bits):
    """fp16 [rows][T][128]: every (32-token group, channel) is zero + k/16 with k covering
    0..2^b-1, so the outer quantizer stores scale 1/16 and decodes exactly."""
    N = (1 << bits) - 1
    k = rng.integers(0, N + 1, (rows, T // 32, 32, 128))
    k[:, :, 0, :] = 0
    k[:, :, 1, :] = N
    m = rng.integers(-40, 40, (rows, T // 32, 1, 128)) / 16.0
    return _f16((m + k / 16.0).reshape(rows, T, 128))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_outer_attention_on_exact_grid_equals_window_attention(oracle_mod, bits):
    O = oracle_mod
    rng = np.random.default_rng(40 + bits)
    fmt = O.Format(bits, 128, False)
    B, Hq, Hkv, n_packed, n_res = 2, 8, 2, 256, 9
    rows = B * Hkv
    ks, vs = _grid_block(rng, rows, n_packed, bits), _grid_block(rng, rows, n_packed, bits)
    kp, vp = O.quantize_pack_outer(fmt, ks), O.quantize_pack_outer(fmt, vs)
    kr = _f16(rng.standard_normal((B, Hkv, 16, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, 16, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    got = O.attention_outer(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, sm=SM)
    kw = np.zeros((B, Hkv, n_packed + n_res, 128), np.float16)
    vw = np.zeros_like(kw)
    kw[:, :, :n_packed] = ks.reshape(B, Hkv, n_packed, 128)
    vw[:, :, :n_packed] = vs.reshape(B, Hkv, n_packed, 128)
    kw[:, :, n_packed:] = kr[:, :, :n_res]
    vw[:, :, n_packed:] = vr[:, :, :n_res]
    empty = np.zeros((rows, 0), np.uint8)
    ref = O.attention(O.Format(bits), q, Hkv, empty, empty, 0, kw, vw, n_packed + n_res, sm=SM)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("S_", [1, 4, 7])
def test_outer_split_partials_merge(oracle_mod, S_):
    O = oracle_mod
    rng = np.random.default_rng(S_)
    fmt = O.Format(3, 128, False)
    B, Hq, Hkv, n_packed, n_res = 1, 4, 1, 384, 20
    ks = _f16(rng.standard_normal((Hkv, n_packed, 128)))
    vs = _f16(rng.standard_normal((Hkv, n_packed, 128)))
    kp, vp = O.quantize_pack_outer(fmt, ks), O.quantize_pack_outer(fmt, vs)
    kr = _f16(rng.standard_normal((B, Hkv, 32, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, 32, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)) * 2)
    one = O.attention_outer(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, sm=SM)
    po, pl = O.split_attention_outer(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, S=S_, sm=SM)
    assert np.max(np.abs(O.combine(po, pl) - one)) < 1e-12


def test_inner_and_outer_error_on_outlier_channels(oracle_mod):
    """Record the two groupings' attention error against unquantized attention on the
    tiny workload (K channels 3 and 77 eight times the rest); both stay finite and both
    shrink from 2 to 4 bits."""
    O = oracle_mod
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    kps, vps = x.packed_src()
    kps = np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))
    vps = np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))
    kr, vr = x.residual()
    empty = np.zeros((rows, 0), np.uint8)
    ref = O.attention(O.Format(4), x.q, wl.Hkv, empty, empty, 0, x.k, x.v, wl.L, sm=SM)
    errs = {}
    for bits in (2, 3, 4):
        fmt = O.Format(bits, 128, False)
        inner = O.attention(fmt, x.q, wl.Hkv, O.quantize_pack(fmt, kps), O.quantize_pack(fmt, vps),
                            wl.n_packed, kr, vr, wl.n_res, sm=SM)
        outer = O.attention_outer(fmt, x.q, wl.Hkv, O.quantize_pack_outer(fmt, kps),
                                  O.quantize_pack_outer(fmt, vps), wl.n_packed, kr, vr,
                                  wl.n_res, sm=SM)
        e = [float(np.linalg.norm(a - ref) / np.linalg.norm(ref)) for a in (inner, outer)]
        errs[bits] = e
        print(f"[grouping] bits={bits} rel-L2 inner {e[0]:.4f} outer {e[1]:.4f}")
        assert all(np.isfinite(e))
    assert errs[4][0] < errs[2][0] and errs[4][1] < errs[2][1]
