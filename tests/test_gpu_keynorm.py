"""GPU parity of key-channel normalization (kvq_key_norm, kvq_channel_scale,
kvq_decode_attention_knorm) against the CPU oracle.

Bar: bit-exact for the factors and the scaled fp16 vectors (both sides do one binary32
operation then round to nearest even; the square root and the division are correctly
rounded on both); the knorm decode's partials equal, bit for bit, those of kvq_channel_scale
on q followed by kvq_decode_attention; the whole normalized pipeline (factors, scaled keys,
packed cache, decode, combine) meets the attention bar of the other decode tests against
the oracle's pipeline."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _gpu_key_norm(k16, n_tokens=None, pad_tok=0, pad_row=0):
    """kvq_key_norm over k16[rows][T][128] placed in a buffer with padded strides."""
    from gpu_common import DEV, dev
    rows, T, d = k16.shape
    n = T if n_tokens is None else n_tokens
    ts = d + pad_tok
    buf = np.full((rows, T + pad_row, ts), np.float16(1000.0), np.float16)   # padding is loud
    buf[:, :T, :d] = k16
    kd = dev(buf)
    norm = torch.full((rows, d), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_key_norm(kd, rows, n, (T + pad_row) * ts, ts, d, norm)
    torch.cuda.synchronize()
    return norm.cpu().numpy()


def _gpu_scale(x16, norm, rows_per_norm=1, multiply=False, pad_tok=0):
    from gpu_common import dev
    rows, T, d = x16.shape
    ts = d + pad_tok
    buf = np.zeros((rows, T, ts), np.float16)
    buf[:, :, :d] = x16
    xd = dev(buf)
    yd = torch.full_like(xd, float("nan"))
    K.kvq_channel_scale(xd, rows, T, T * ts, ts, d, dev(np.asarray(norm, np.float32)),
                        rows_per_norm, K.KVQ_SCALE_MULTIPLY if multiply else K.KVQ_SCALE_DIVIDE,
                        yd, T * ts, ts)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    if pad_tok:
        assert np.all(np.isnan(y[:, :, d:])), "padding channels were written"
    return y[:, :, :d]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def _assert_same_f16(got_bits, ref_bits, x=None, norm=None):
    """Bit-exact, with the first differing elements in the message."""
    got_bits, ref_bits = np.asarray(got_bits), np.asarray(ref_bits)
    bad = np.argwhere(got_bits != ref_bits)
    if len(bad) == 0:
        return
    lines = [f"{len(bad)} of {got_bits.size} differ"]
    for idx in bad[:8]:
        t = tuple(idx)
        xs = "" if x is None else f" x={float(np.asarray(x)[t]):.9g}"
        ns = "" if norm is None else f" norm={float(norm[t[0], t[-1]]):.9g}"
        lines.append(f"  {t}:{xs}{ns} got=0x{int(got_bits[t]):04x} ref=0x{int(ref_bits[t]):04x}")
    raise AssertionError("\n".join(lines))


@pytest.mark.parametrize("T,pad_tok,pad_row,seed", [
    (1024, 0, 0, 0),       # several 256-token chunks
    (300, 8, 5, 1),        # ragged last chunk, strided tokens and rows
    (1, 0, 0, 2),
    (257, 0, 3, 3),
])
def test_key_norm_matches_oracle(oracle_mod, T, pad_tok, pad_row, seed):
    rng = np.random.default_rng(seed)
    rows = 6
    print(f"[key_norm] rows={rows} T={T} pad_tok={pad_tok} pad_row={pad_row}", flush=True)
    k = _f16(rng.standard_normal((rows, T, 128)) * rng.uniform(0.001, 30.0, (rows, 1, 128)))
    k[1, :, 5] = 0                                   # all-zero channel -> 1
    k[2, :, 9] = np.float16(-0.0)                    # negative zeros count as zero
    k[3, :, 17] = np.float16(6e-8)                   # subnormal maximum
    k[4, T // 2, 40] = np.float16(-60000.0)          # large negative outlier
    got = _gpu_key_norm(k, pad_tok=pad_tok, pad_row=pad_row)
    ref = oracle_mod.key_norm(k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert got[1, 5] == 1.0 and got[2, 9] == 1.0


def test_key_norm_of_every_fp16_magnitude(oracle_mod):
    """Every finite fp16 magnitude 0..65504 is a channel maximum once: the device square
    root (and the 1 for 0) agrees with the CPU's correctly rounded one on all of them."""
    mags = np.arange(0, 0x7c00, dtype=np.uint16)                     # 31744 values
    rows = (len(mags) + 127) // 128
    m = np.zeros(rows * 128, np.uint16)
    m[:len(mags)] = mags
    k = np.zeros((rows, 3, 128), np.uint16)
    k[:, 0, :] = m.reshape(rows, 128)
    k[:, 1, :] = (m.reshape(rows, 128) >> 1) | 0x8000                # smaller, negative
    k = k.view(np.float16)
    print(f"[key_norm] exhaustive rows={rows}", flush=True)
    got = _gpu_key_norm(k)
    ref = oracle_mod.key_norm(k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_key_norm_of_no_tokens_is_one():
    from gpu_common import DEV
    norm = torch.full((3, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_key_norm(None, 3, 0, 0, 128, 128, norm)
    torch.cuda.synchronize()
    assert torch.all(norm == 1.0)


@pytest.mark.parametrize("multiply", [False, True])
def test_channel_scale_every_fp16_value(oracle_mod, multiply):
    """All 63488 finite fp16 values against norms spread over 2^-12 .. 2^12 (quotients and
    products that overflow to inf and fall into subnormals included): bit-exact."""
    vals = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = vals[(vals & 0x7c00) != 0x7c00]                           # finite only
    T = (len(vals) + 127) // 128
    x = np.zeros(T * 128, np.uint16)
    x[:len(vals)] = vals
    rows = 4
    x = np.broadcast_to(x.reshape(1, T, 128), (rows, T, 128)).copy().view(np.float16)
    rng = np.random.default_rng(7)
    norm = (2.0 ** rng.uniform(-12, 12, (rows, 128))).astype(np.float32)
    norm[0, :4] = [1.0, 3.0, 1.0 / 3.0, np.float32(np.sqrt(np.float32(2.0)))]
    print(f"[channel_scale] exhaustive multiply={multiply} T={T}", flush=True)
    got = _gpu_scale(x, norm, multiply=multiply)
    ref = oracle_mod.channel_scale(x, norm, multiply=multiply)
    _assert_same_f16(_bits(got), ref, x, norm)


@pytest.mark.parametrize("T,pad_tok,rpn,seed", [(1000, 0, 1, 0), (77, 16, 1, 1), (1, 0, 4, 2),
                                                (130, 8, 2, 3)])
@pytest.mark.parametrize("multiply", [False, True])
def test_channel_scale_matches_oracle(oracle_mod, T, pad_tok, rpn, seed, multiply):
    rng = np.random.default_rng(seed)
    rows = 8
    print(f"[channel_scale] rows={rows} T={T} pad_tok={pad_tok} rows_per_norm={rpn} "
          f"multiply={multiply}", flush=True)
    x = _f16(rng.standard_normal((rows, T, 128)) * rng.uniform(0.01, 50.0, (rows, 1, 128)))
    norm = oracle_mod.key_norm(_f16(rng.standard_normal((rows // rpn, 64, 128)) *
                                    rng.uniform(0.01, 50.0, (rows // rpn, 1, 128))))
    got = _gpu_scale(x, norm, rows_per_norm=rpn, multiply=multiply, pad_tok=pad_tok)
    ref = oracle_mod.channel_scale(x, norm, rows_per_norm=rpn, multiply=multiply)
    _assert_same_f16(_bits(got), ref, x, np.repeat(norm, rpn, axis=0))


def test_channel_scale_in_place_and_into_a_window_slot(oracle_mod):
    """In place (x == y), and a new key scaled straight into slot 37 of a residual window
    (the other slots untouched); n_tokens == 0 writes nothing."""
    from gpu_common import dev
    rng = np.random.default_rng(11)
    B, Hkv, cap = 2, 4, 128
    rows = B * Hkv
    norm = (2.0 ** rng.uniform(-3, 3, (rows, 128))).astype(np.float32)
    nd = dev(norm)
    x = _f16(rng.standard_normal((rows, 200, 128)) * 4)
    xd = dev(x)
    K.kvq_channel_scale(xd, rows, 200, 200 * 128, 128, 128, nd, 1, K.KVQ_SCALE_DIVIDE, xd,
                        200 * 128, 128)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(xd.cpu().numpy()), oracle_mod.channel_scale(x, norm))

    win = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    wd = dev(win)
    knew = _f16(rng.standard_normal((B, Hkv, 128)) * 5)
    slot = 37
    K.kvq_channel_scale(dev(knew), rows, 1, 128, 128, 128, nd, 1, K.KVQ_SCALE_DIVIDE,
                        wd[:, :, slot], cap * 128, 128)
    K.kvq_channel_scale(dev(knew), rows, 0, 128, 128, 128, nd, 1, K.KVQ_SCALE_DIVIDE,
                        wd[:, :, 0], cap * 128, 128)
    torch.cuda.synchronize()
    w = wd.cpu().numpy()
    ref = oracle_mod.channel_scale(knew.reshape(rows, 1, 128), norm).reshape(B, Hkv, 128)
    assert np.array_equal(_bits(w[:, :, slot]), ref)
    keep = np.ones(cap, bool)
    keep[slot] = False
    assert np.array_equal(_bits(w[:, :, keep]), _bits(win[:, :, keep]))


def _packed_case(rng, bits, hybrid, B, Hq, Hkv, n_packed, n_res):
    from gpu_common import dev, gpu_quantize
    rows = B * Hkv
    fmt = K.Format(bits, 128, hybrid)
    k = _f16(rng.standard_normal((rows, n_packed, 128)))
    v = _f16(rng.standard_normal((rows, n_packed, 128)))
    kp = gpu_quantize(fmt, k) if n_packed else None
    vp = gpu_quantize(fmt, v) if n_packed else None
    kr = dev(_f16(rng.standard_normal((B, Hkv, 128, 128))))
    vr = dev(_f16(rng.standard_normal((B, Hkv, 128, 128))))
    q = _f16(rng.standard_normal((B, Hq, 128)) * 3)
    norm = (2.0 ** rng.uniform(-4, 4, (rows, 128))).astype(np.float32)
    return fmt, kp, vp, kr, vr, q, norm


@pytest.mark.parametrize("bits,hybrid,B,Hq,Hkv,n_packed,n_res,S_", [
    (4, False, 1, 8, 2, 896, 128, 5),
    (4, False, 2, 32, 8, 1024, 17, 3),
    (2, True, 1, 16, 1, 512, 0, 2),
    (3, False, 1, 4, 4, 384, 64, 1),       # one query head per kv head
    (4, False, 1, 16, 4, 0, 100, 1),       # residual window only
])
def test_decode_knorm_equals_scaled_q_then_decode(bits, hybrid, B, Hq, Hkv, n_packed, n_res,
                                                  S_):
    from gpu_common import DEV, dev
    rng = np.random.default_rng(bits * 100 + Hq)
    print(f"[decode_knorm] bits={bits} hybrid={hybrid} B={B} Hq={Hq} Hkv={Hkv} "
          f"n_packed={n_packed} n_res={n_res} S={S_}", flush=True)
    fmt, kp, vp, kr, vr, q, norm = _packed_case(rng, bits, hybrid, B, Hq, Hkv, n_packed, n_res)
    qd, nd = dev(q), dev(norm)
    stride = kp.shape[1] if kp is not None else 0

    def run(entry, qq, extra=()):
        po = torch.full((B, Hq, S_, 128), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, S_), float("nan"), dtype=torch.float32, device=DEV)
        entry(fmt, qq, *extra, B, Hq, Hkv, kp, vp, stride, n_packed, kr, vr, 128, n_res, SM, S_,
              po, pl)
        return po, pl

    qs = torch.empty_like(qd)
    K.kvq_channel_scale(qd, B * Hq, 1, 128, 128, 128, nd, Hq // Hkv, K.KVQ_SCALE_MULTIPLY, qs,
                        128, 128)
    po_ref, pl_ref = run(K.kvq_decode_attention, qs)
    po, pl = run(K.kvq_decode_attention_knorm, qd, (nd,))
    torch.cuda.synchronize()
    assert torch.equal(po, po_ref) and torch.equal(pl, pl_ref)
    # and the factors were applied at all
    po_plain, _ = run(K.kvq_decode_attention, qd)
    torch.cuda.synchronize()
    assert not torch.equal(po, po_plain)


@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, False), (2, True)])
def test_normalized_pipeline_matches_oracle(oracle_mod, bits, hybrid):
    """tiny workload (K channels 3 and 77 eight times the rest): factors from the prefill
    keys, keys scaled and packed, window keys scaled, decode with q multiplied in the
    kernel, combine -- all on the GPU -- against the same steps in the oracle."""
    from gpu_common import DEV, assert_close, dev, gpu_quantize
    O = oracle_mod
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    kps, vps = x.packed_src()
    kps = np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))
    vps = np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))
    kr, vr = x.residual()
    print(f"[knorm pipeline] bits={bits} hybrid={hybrid} tiny", flush=True)

    # oracle
    n_ref = O.key_norm(kps)
    kn_ref = O.channel_scale(kps, n_ref).view(np.float16)
    krn_ref = O.channel_scale(kr.reshape(rows, -1, 128), n_ref).view(np.float16).reshape(kr.shape)
    qn_ref = O.channel_scale(x.q.reshape(wl.B * wl.Hq, 1, 128), n_ref, rows_per_norm=wl.gq,
                             multiply=True).view(np.float16).reshape(x.q.shape)
    kp_ref = O.quantize_pack(ofmt, kn_ref)
    vp_ref = O.quantize_pack(ofmt, vps)
    ref = O.attention(ofmt, qn_ref, wl.Hkv, kp_ref, vp_ref, wl.n_packed, krn_ref, vr, wl.n_res,
                      sm=SM)

    # GPU
    kd = dev(kps)
    nd = torch.empty((rows, 128), dtype=torch.float32, device=DEV)
    K.kvq_key_norm(kd, rows, wl.n_packed, wl.n_packed * 128, 128, 128, nd)
    K.kvq_channel_scale(kd, rows, wl.n_packed, wl.n_packed * 128, 128, 128, nd, 1,
                        K.KVQ_SCALE_DIVIDE, kd, wl.n_packed * 128, 128)
    krd = dev(kr)
    cap = kr.shape[2]
    K.kvq_channel_scale(krd, rows, wl.n_res, cap * 128, 128, 128, nd, 1, K.KVQ_SCALE_DIVIDE,
                        krd, cap * 128, 128)
    kp = torch.zeros((rows, wl.n_packed // 128 * fmt.block_bytes), dtype=torch.uint8, device=DEV)
    K.kvq_quantize_pack(fmt, kd, rows, wl.n_packed, wl.n_packed * 128, 128, kp, kp.shape[1], 0)
    vp = gpu_quantize(fmt, vps)
    S_ = 4
    po = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_knorm(fmt, dev(x.q), nd, wl.B, wl.Hq, wl.Hkv, kp, vp, kp.shape[1],
                                 wl.n_packed, krd, dev(vr), cap, wl.n_res, SM, S_, po, pl)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_combine(po, pl, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F32)
    torch.cuda.synchronize()

    assert np.array_equal(nd.cpu().numpy().view(np.uint32), n_ref.view(np.uint32))
    assert np.array_equal(_bits(kd.cpu().numpy()), _bits(kn_ref))
    assert np.array_equal(_bits(krd.cpu().numpy()), _bits(krn_ref))
    assert np.array_equal(kp.cpu().numpy(), kp_ref)
    assert_close(out.cpu().numpy(), ref, "normalized attention")
