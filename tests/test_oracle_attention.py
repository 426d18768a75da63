"""Pins of the oracle's decode attention and split/combine.

- all tokens in the fp16 residual window: the textbook softmax(q K^T / sqrt(d)) V, here
  torch.nn.functional.scaled_dot_product_attention in fp64 on the CPU;
- closed forms: one token -> its value; q = 0 -> mean of the values; constant V -> V;
- brute force on tiny shapes: the packed cache dequantized by an independent Python
  reader of the block format (big-int code unpacking), attention in numpy fp64, with
  several kv heads so the GQA head mapping is exercised;
- the split-K partials merged by the combine equal the one-pass result.
"""
import numpy as np
import pytest
import torch

import synth_inputs as S

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _py_dequant_row(packed_row, bits, hybrid, n_tokens, d=128):
    """Independent reader of the packed block format -> fp64 [n_tokens][d]."""
    ng = d // 32
    gb = 4 * bits
    codes_bytes = 128 * d * bits // 8
    sz_off = codes_bytes
    bb = codes_bytes + 128 * ng * 4 + (64 if hybrid else 0)
    out = np.zeros((n_tokens, d))
    raw = packed_row.tobytes()
    for t in range(n_tokens):
        blk = raw[(t // 128) * bb:(t // 128 + 1) * bb]
        tb = t % 128
        for g in range(ng):
            w = int.from_bytes(blk[tb * ng * gb + g * gb: tb * ng * gb + (g + 1) * gb], "little")
            so = sz_off + (tb * ng + g) * 4
            s = float(np.frombuffer(blk[so:so + 2], np.float16)[0])
            z = float(np.frombuffer(blk[so + 2:so + 4], np.float16)[0])
            for i in range(32):
                out[t, 32 * g + i] = z + ((w >> (bits * i)) & ((1 << bits) - 1)) * s
    return out


def _np_attention(q, K, V, gq, sm):
    """q [B][Hq][d], K,V [B][Hkv][n][d] fp64 -> out [B][Hq][d]."""
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kv = h // gq
            lg = sm * (K[b, kv] @ q[b, h])
            p = np.exp(lg - lg.max())
            out[b, h] = (p[:, None] * V[b, kv]).sum(0) / p.sum()
    return out


def test_all_residual_equals_sdpa(oracle_mod):
    O = oracle_mod
    fmt = O.Format(4)
    rng = np.random.default_rng(11)
    B, Hq, Hkv, n = 2, 8, 2, 100
    q = _f16(rng.standard_normal((B, Hq, 128)))
    kr = _f16(rng.standard_normal((B, Hkv, 128, 128)) * 2)
    vr = _f16(rng.standard_normal((B, Hkv, 128, 128)))
    empty = np.zeros((B * Hkv, 0), np.uint8)
    out = O.attention(fmt, q, Hkv, empty, empty, 0, kr, vr, n, sm=SM)
    gq = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).unsqueeze(2)
    kt = torch.from_numpy(kr[:, :, :n].astype(np.float64)).repeat_interleave(gq, dim=1)
    vt = torch.from_numpy(vr[:, :, :n].astype(np.float64)).repeat_interleave(gq, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM).squeeze(2)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_single_token_returns_its_value(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(12)
    q = _f16(rng.standard_normal((1, 4, 128)))
    kr = _f16(rng.standard_normal((1, 1, 128, 128)))
    vr = _f16(rng.standard_normal((1, 1, 128, 128)))
    empty = np.zeros((1, 0), np.uint8)
    out = O.attention(O.Format(4), q, 1, empty, empty, 0, kr, vr, 1, sm=SM)
    assert np.array_equal(out, np.broadcast_to(vr[0, 0, 0].astype(np.float64), (1, 4, 128)))


@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, False), (2, True)])
def test_zero_query_averages_values(oracle_mod, bits, hybrid):
    O = oracle_mod
    fmt = O.Format(bits, 128, hybrid)
    rng = np.random.default_rng(13)
    src = _f16(rng.standard_normal((2, 256, 128)))
    kp = O.quantize_pack(fmt, src)
    vp = O.quantize_pack(fmt, _f16(rng.standard_normal((2, 256, 128))))
    kr = _f16(rng.standard_normal((1, 2, 128, 128)))
    vr = _f16(rng.standard_normal((1, 2, 128, 128)))
    q = np.zeros((1, 4, 128), np.float16)
    out = O.attention(fmt, q, 2, kp, vp, 256, kr, vr, 50, sm=SM)
    vdeq = O.dequant(fmt, vp, 256)
    for h in range(4):
        kv = h // 2
        allv = np.concatenate([vdeq[kv], vr[0, kv, :50].astype(np.float64)])
        assert np.max(np.abs(out[0, h] - allv.mean(0))) < 1e-12


def test_constant_values_give_that_value(oracle_mod):
    O = oracle_mod
    fmt = O.Format(4)
    rng = np.random.default_rng(14)
    kp = O.quantize_pack(fmt, _f16(rng.standard_normal((1, 128, 128))))
    vrow = _f16(rng.standard_normal(128))
    vsrc = np.broadcast_to(vrow, (1, 128, 128)).copy()
    vp = O.quantize_pack(fmt, vsrc)
    q = _f16(rng.standard_normal((1, 2, 128)) * 3)
    out = O.attention(fmt, q, 1, kp, vp, 128, sm=SM)
    # constant columns quantize exactly? no: each token's group is quantized along head_dim,
    # so every token holds the same reconstruction; the attention returns that row
    vhat = O.dequant(fmt, vp, 1)[0, 0]
    assert np.max(np.abs(out[0] - vhat)) < 1e-12


@pytest.mark.parametrize("bits,hybrid,Hq,Hkv,n_packed,n_res", [
    (4, False, 4, 1, 128, 0),
    (4, False, 8, 2, 256, 33),
    (3, False, 4, 4, 128, 1),
    (2, True, 8, 2, 128, 127),
    (2, False, 4, 1, 384, 128),
    (4, True, 2, 2, 128, 3),
])
def test_brute_force_tiny(oracle_mod, bits, hybrid, Hq, Hkv, n_packed, n_res):
    O = oracle_mod
    fmt = O.Format(bits, 128, hybrid)
    rng = np.random.default_rng(15 + bits + Hq + n_res)
    B = 2
    ksrc = _f16(rng.standard_t(5, size=(B * Hkv, n_packed, 128)))
    vsrc = _f16(rng.standard_normal((B * Hkv, n_packed, 128)) * 2)
    kp = O.quantize_pack(fmt, ksrc)
    vp = O.quantize_pack(fmt, vsrc)
    kr = _f16(rng.standard_normal((B, Hkv, 128, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, 128, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    out = O.attention(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, sm=SM)
    K = np.zeros((B, Hkv, n_packed + n_res, 128))
    V = np.zeros_like(K)
    for b in range(B):
        for kv in range(Hkv):
            row = b * Hkv + kv
            K[b, kv, :n_packed] = _py_dequant_row(kp[row], bits, hybrid, n_packed)
            V[b, kv, :n_packed] = _py_dequant_row(vp[row], bits, hybrid, n_packed)
            K[b, kv, n_packed:] = kr[b, kv, :n_res]
            V[b, kv, n_packed:] = vr[b, kv, :n_res]
    ref = _np_attention(q.astype(np.float64), K, V, Hq // Hkv, SM)
    assert np.max(np.abs(out - ref)) < 1e-11


@pytest.mark.parametrize("n_packed,n_res,S", [
    (384, 128, 1), (384, 128, 2), (384, 128, 5), (384, 0, 4), (0, 77, 3),
    (128, 5, 9), (896, 128, 7), (256, 128, 64)])
def test_split_combine_equals_one_pass(oracle_mod, n_packed, n_res, S):
    O = oracle_mod
    fmt = O.Format(4)
    rng = np.random.default_rng(16)
    B, Hq, Hkv = 1, 4, 2
    kp = O.quantize_pack(fmt, _f16(rng.standard_normal((B * Hkv, n_packed, 128))))
    vp = O.quantize_pack(fmt, _f16(rng.standard_normal((B * Hkv, n_packed, 128))))
    if n_packed == 0:
        kp = vp = np.zeros((B * Hkv, 0), np.uint8)
    kr = _f16(rng.standard_normal((B, Hkv, 128, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, 128, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)) * 2)
    one = O.attention(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, sm=SM)
    po, pl = O.split_attention(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, S=S, sm=SM)
    assert np.max(np.abs(O.combine(po, pl) - one)) < 1e-12
    # every token is in exactly one split
    cover = np.zeros(n_packed + n_res, int)
    for s in range(S):
        lo, hi = O.split_range(n_packed, n_res, S, s)
        cover[lo:hi] += 1
        if hi <= lo:
            assert np.all(pl[..., s] == -np.inf) and np.all(po[..., s, :] == 0)
    assert np.all(cover == 1)


def test_combine_closed_form(oracle_mod):
    """Two splits with lse a, b: weights e^a/(e^a+e^b), e^b/(e^a+e^b)."""
    O = oracle_mod
    po = np.zeros((1, 1, 3, 128))
    po[0, 0, 0] = 1.0
    po[0, 0, 1] = 3.0
    pl = np.array([[[np.log(1.0), np.log(3.0), -np.inf]]])
    out = O.combine(po, pl)
    assert np.max(np.abs(out - 2.5)) < 1e-15


def test_workload_recipe_shapes():
    for name, wl in S.WORKLOADS.items():
        assert wl.Hq % wl.Hkv == 0 and wl.n_packed % 128 == 0
    assert S.WORKLOADS["llama8b_32k"].step_bytes() == 42303488
    assert S.WORKLOADS["batch8_2bit_hybrid"].n_packed == 32640
    x = S.make_inputs("tiny")
    kp, vp = x.packed_src()
    kr, vr = x.residual()
    assert kp.shape == (1, 2, 896, 128) and kr.shape == (1, 2, 128, 128)
    assert np.array_equal(kr[:, :, :], x.k[:, :, 896:])
    y = S.make_inputs("batch8_2bit_hybrid", L=512, B=1)
    kp, vp = y.packed_src()
    kr, vr = y.residual()
    assert kp.shape[2] == 384
    assert np.array_equal(kr[:, :, :32], y.k[:, :, :32])
    assert np.array_equal(kr[:, :, 32:], y.k[:, :, 512 - 96:])
    assert np.array_equal(kp, y.k[:, :, 32:32 + 384])
