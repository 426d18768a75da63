"""Pins of the oracle's key-channel normalization (InnerQ page, sec. 2.4): per (row,
channel) norm = sqrt(max |K|) over the prefill tokens, keys divided by it, queries
multiplied by it. Checked against values fixed by arithmetic, the range property the page
states, exact softmax invariance where the scaling is exact, a rounding bound where it is
not, and the quantization-error reduction the step exists for."""
import numpy as np
import pytest

import synth_inputs as S

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def test_norm_of_perfect_squares_and_zero_channel(oracle_mod):
    O = oracle_mod
    k = np.zeros((2, 5, 128), np.float16)
    k[0, :, 0] = [-9, 4, 1, 0, 2]          # max |.| = 9   -> 3
    k[0, :, 1] = [0.25, -16, 3, 1, 1]      # 16            -> 4
    k[1, :, 5] = [-0.0625, 0, 0, 0, 0]     # 1/16          -> 1/4
    n = O.key_norm(k)
    assert n[0, 0] == 3.0 and n[0, 1] == 4.0 and n[1, 5] == 0.25
    # all-zero channels are left alone
    assert n[0, 2] == 1.0 and n[1, 0] == 1.0
    kk = O.channel_scale(k, n).view(np.float16)
    assert np.array_equal(kk[0, :, 2], k[0, :, 2])
    # power-of-two norms scale exactly
    assert np.array_equal(kk[0, :, 1].astype(np.float32), k[0, :, 1].astype(np.float32) / 4)


def test_scaled_keys_peak_at_the_square_root(oracle_mod):
    """max_t |K'[t][i]| = max|K| / sqrt(max|K|) = sqrt(max|K|) = norm_i, up to the fp16
    rounding of the quotient (a key multiplied instead of divided would peak at the
    1.5th power)."""
    O = oracle_mod
    rng = np.random.default_rng(0)
    k = _f16(rng.standard_normal((3, 200, 128)) * rng.uniform(0.01, 40.0, (3, 1, 128)))
    n = O.key_norm(k)
    kk = O.channel_scale(k, n).view(np.float16).astype(np.float64)
    peak = np.abs(kk).max(axis=1)
    assert np.allclose(peak, n, rtol=2.0 ** -11, atol=0)


def _attn(O, q, k, v, Hkv):
    """fp64 attention over fp16 q, k, v with every token unquantized."""
    rows = k.shape[0] * k.shape[1]
    empty = np.zeros((rows, 0), np.uint8)
    return O.attention(O.Format(4), q, Hkv, empty, empty, 0, k, v, k.shape[2], sm=SM)


def test_softmax_invariance_with_exact_scalings(oracle_mod):
    """With per-channel maxima of 4^j the norms are powers of two, so q' . k' = q . k
    exactly and the attention output is unchanged to the last bit of fp64."""
    O = oracle_mod
    rng = np.random.default_rng(1)
    B, Hq, Hkv, L = 1, 8, 2, 96
    mags = 4.0 ** rng.integers(-2, 4, (B * Hkv, 1, 128))
    u = rng.uniform(-1, 1, (B * Hkv, L, 128))
    u[:, 0, :] = 1.0                                  # pin the maximum at exactly 4^j
    k = _f16(u * mags)
    v = _f16(rng.standard_normal((B * Hkv, L, 128)))
    q = _f16(rng.uniform(-1, 1, (B, Hq, 128)))
    n = O.key_norm(k)
    assert np.all(np.log2(n) == np.round(np.log2(n)))
    kq = O.channel_scale(k, n).view(np.float16)
    qq = O.channel_scale(q.reshape(B * Hq, 1, 128), n, rows_per_norm=Hq // Hkv,
                         multiply=True).view(np.float16).reshape(B, Hq, 128)
    ref = _attn(O, q, k.reshape(B, Hkv, L, 128), v.reshape(B, Hkv, L, 128), Hkv)
    got = _attn(O, qq, kq.reshape(B, Hkv, L, 128), v.reshape(B, Hkv, L, 128), Hkv)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_query_rows_use_their_kv_head_norm(oracle_mod):
    O = oracle_mod
    B, Hq, Hkv = 2, 8, 2
    n = (np.arange(B * Hkv * 128, dtype=np.float32).reshape(B * Hkv, 128) % 7 + 1) * 0.5
    q = np.ones((B * Hq, 1, 128), np.float16)
    qq = O.channel_scale(q, n, rows_per_norm=Hq // Hkv, multiply=True).view(np.float16)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(qq[b * Hq + h, 0].astype(np.float32), n[b * Hkv + h // (Hq // Hkv)])


def test_logits_move_by_at_most_the_fp16_rounding(oracle_mod):
    """General norms: q'_i and k'_i are each within 2^-11 (relative) of q_i * n_i and
    k_i / n_i, so |q' . k' - q . k| <= sum_i |q_i k_i| (2^-10 + 2^-22)."""
    O = oracle_mod
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    k = x.k.reshape(rows, wl.L, 128)
    n = O.key_norm(k)
    kk = O.channel_scale(k, n).view(np.float16).astype(np.float64)
    qq = O.channel_scale(x.q.reshape(wl.B * wl.Hq, 1, 128), n, rows_per_norm=wl.gq,
                         multiply=True).view(np.float16).astype(np.float64)
    qf = x.q.reshape(wl.B * wl.Hq, 128).astype(np.float64)
    kf = k.astype(np.float64)
    for h in range(wl.Hq):
        r = h // wl.gq
        lhs = np.abs(kk[r] @ qq[h, 0] - kf[r] @ qf[h])
        bound = (np.abs(kf[r]) @ np.abs(qf[h])) * (2.0 ** -10 + 2.0 ** -22)
        assert np.all(lhs <= bound + 1e-300)


def test_outlier_channels_are_compressed_to_the_square_root(oracle_mod):
    """tiny workload: K channels 3 and 77 are 8x the rest; after normalization their peak
    is sqrt(8) ~ 2.83x the others' (the spread is square-rooted)."""
    O = oracle_mod
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    k = x.k.reshape(wl.B * wl.Hkv, wl.L, 128)
    before = np.abs(k.astype(np.float64)).max(axis=1)
    kk = O.channel_scale(k, O.key_norm(k)).view(np.float16).astype(np.float64)
    after = np.abs(kk).max(axis=1)
    others = [c for c in range(128) if c not in (3, 77)]
    rb = before[:, [3, 77]].mean() / np.median(before[:, others])
    ra = after[:, [3, 77]].mean() / np.median(after[:, others])
    assert 6.0 < rb < 10.0
    assert abs(ra - np.sqrt(rb)) < 0.05 * np.sqrt(rb)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_normalization_cuts_quantized_attention_error_on_outliers(oracle_mod, bits):
    """What the step is for: on a cache with outlier key channels, quantizing K / norm
    (and using q * norm) gives attention closer to the unquantized fp64 attention than
    quantizing K as is. Everything here is the oracle (quantizer + fp64 attention)."""
    O = oracle_mod
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    fmt = O.Format(bits)
    kps, vps = x.packed_src()
    kps = np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))
    vps = np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))
    kr, vr = x.residual()
    ref = _attn(O, x.q, x.k, x.v, wl.Hkv)
    vp = O.quantize_pack(fmt, vps)

    plain = O.attention(fmt, x.q, wl.Hkv, O.quantize_pack(fmt, kps), vp, wl.n_packed, kr, vr,
                        wl.n_res, sm=SM)
    n = O.key_norm(kps)                                  # prefill statistics
    kn = O.channel_scale(kps, n).view(np.float16)
    krn = O.channel_scale(kr.reshape(rows, 128, 128), n).view(np.float16).reshape(kr.shape)
    qn = O.channel_scale(x.q.reshape(wl.B * wl.Hq, 1, 128), n, rows_per_norm=wl.gq,
                         multiply=True).view(np.float16).reshape(x.q.shape)
    normed = O.attention(fmt, qn, wl.Hkv, O.quantize_pack(fmt, kn), vp, wl.n_packed, krn, vr,
                         wl.n_res, sm=SM)
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    e_norm = np.linalg.norm(normed - ref) / np.linalg.norm(ref)
    print(f"[key norm] bits={bits} rel-L2 error vs unquantized: plain {e_plain:.4e} "
          f"normalized {e_norm:.4e}")
    assert e_norm < e_plain
