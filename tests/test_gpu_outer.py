"""GPU parity of the outer-dimension (KIVI-style) comparison path (kvq_quantize_pack_outer,
kvq_decode_attention_outer) against the CPU oracle: packed bytes bit-exact; partials and
combined output within the attention bar (max-abs 2e-3, rel-L2 1e-3)."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_outer_quantize_bytes(oracle_mod, bits):
    from gpu_common import DEV, dev
    O = oracle_mod
    rng = np.random.default_rng(bits)
    rows, T = 3, 384
    x = _f16(rng.standard_normal((rows, T, 128)) * rng.uniform(0.01, 30, (rows, 1, 128)))
    x[0, :32, 7] = 2.5                      # constant group
    x[1, 32:64, 9] = np.float16(-0.0)       # negative zeros
    x[2, 64:96, 100] = rng.choice([-60000.0, 60000.0, 1e-7], 32)   # huge range
    fmt, ofmt = K.Format(bits), O.Format(bits)
    print(f"[quantize_outer] bits={bits}", flush=True)
    ref = O.quantize_pack_outer(ofmt, x)
    # strided source (tokens padded to 136 halves) written at block 1 of a 4-block row
    pad = np.zeros((rows, T, 136), np.float16)
    pad[:, :, :128] = x
    bb = fmt.block_bytes
    dst = torch.full((rows, 4 * bb), 0xAB, dtype=torch.uint8, device=DEV)
    K.kvq_quantize_pack_outer(fmt, dev(pad), rows, T, T * 136, 136, dst, 4 * bb, 1)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:, bb:4 * bb], ref)
    assert np.all(got[:, :bb] == 0xAB)


def _outer_case(O, rng, bits, B, Hq, Hkv, n_packed, n_res, scale=1.0):
    from gpu_common import DEV, dev
    rows = B * Hkv
    fmt, ofmt = K.Format(bits), O.Format(bits)
    ks = _f16(rng.standard_normal((rows, n_packed, 128)) * scale)
    vs = _f16(rng.standard_normal((rows, n_packed, 128)) * scale)
    kp_ref = O.quantize_pack_outer(ofmt, ks) if n_packed else np.zeros((rows, 0), np.uint8)
    vp_ref = O.quantize_pack_outer(ofmt, vs) if n_packed else np.zeros((rows, 0), np.uint8)
    if n_packed:
        bb = fmt.block_bytes
        kp = torch.empty((rows, n_packed // 128 * bb), dtype=torch.uint8, device=DEV)
        vp = torch.empty_like(kp)
        K.kvq_quantize_pack_outer(fmt, dev(ks), rows, n_packed, n_packed * 128, 128, kp, kp.shape[1], 0)
        K.kvq_quantize_pack_outer(fmt, dev(vs), rows, n_packed, n_packed * 128, 128, vp, vp.shape[1], 0)
    else:
        kp = vp = None
    kr = _f16(rng.standard_normal((B, Hkv, 128, 128)) * scale)
    vr = _f16(rng.standard_normal((B, Hkv, 128, 128)) * scale)
    q = _f16(rng.standard_normal((B, Hq, 128)))
    return fmt, ofmt, kp, vp, kp_ref, vp_ref, kr, vr, q


CASES = [
    # bits, B, Hq, Hkv, n_packed, n_res, S
    (4, 1, 8, 2, 896, 128, 1),
    (4, 1, 8, 2, 896, 128, 7),
    (4, 2, 32, 8, 1024, 37, 5),
    (3, 1, 16, 1, 640, 0, 3),
    (2, 3, 4, 4, 256, 5, 2),
    (4, 1, 12, 2, 384, 1, 4),        # 6 heads per kv head: chunks of 4 and 2
    (2, 1, 8, 1, 0, 70, 1),          # window only
    (4, 1, 8, 2, 16384, 128, 1024),  # the split limit
]


@pytest.mark.parametrize("bits,B,Hq,Hkv,n_packed,n_res,S_", CASES)
def test_outer_decode_matches_oracle(oracle_mod, bits, B, Hq, Hkv, n_packed, n_res, S_):
    from gpu_common import assert_close, dev, gpu_decode
    O = oracle_mod
    rng = np.random.default_rng(n_packed + Hq + bits)
    fmt, ofmt, kp, vp, kp_ref, vp_ref, kr, vr, q = _outer_case(O, rng, bits, B, Hq, Hkv,
                                                               n_packed, n_res)
    print(f"[decode_outer] bits={bits} B={B} Hq={Hq} Hkv={Hkv} n_packed={n_packed} "
          f"n_res={n_res} S={S_}", flush=True)
    out, po, pl = gpu_decode(fmt, dev(q), Hkv, kp, vp, n_packed, dev(kr), dev(vr), n_res, S_,
                             sm=SM, entry=K.kvq_decode_attention_outer)
    torch.cuda.synchronize()
    ref = O.attention_outer(ofmt, q, Hkv, kp_ref, vp_ref, n_packed, kr, vr, n_res, sm=SM)
    assert_close(out.cpu().numpy(), ref, "attention")
    rpo, rpl = O.split_attention_outer(ofmt, q, Hkv, kp_ref, vp_ref, n_packed, kr, vr, n_res,
                                       S=S_, sm=SM)
    gpl, gpo = pl.cpu().numpy(), po.cpu().numpy()
    empty = np.isneginf(rpl)
    assert np.array_equal(np.isneginf(gpl), empty)
    assert np.max(np.abs(gpl[~empty] - rpl[~empty])) < 1e-3
    assert_close(gpo[~empty], rpo[~empty], "partials")


@pytest.mark.slow
def test_outer_decode_full_32k(oracle_mod):
    """The llama8b_32k workload (4 random K channels x10) with outer groups, at the split
    count the benchmark uses: every output against the oracle."""
    from gpu_common import DEV, assert_close, bench_splits, dev
    O = oracle_mod
    wl = S.WORKLOADS["llama8b_32k"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    fmt, ofmt = K.Format(4), O.Format(4)
    kps, vps = x.packed_src()
    kps = np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))
    vps = np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))
    kr, vr = x.residual()
    print("[decode_outer] llama8b_32k full", flush=True)
    bb = fmt.block_bytes
    kp = torch.empty((rows, wl.n_packed // 128 * bb), dtype=torch.uint8, device=DEV)
    vp = torch.empty_like(kp)
    K.kvq_quantize_pack_outer(fmt, dev(kps), rows, wl.n_packed, wl.n_packed * 128, 128, kp, kp.shape[1], 0)
    K.kvq_quantize_pack_outer(fmt, dev(vps), rows, wl.n_packed, wl.n_packed * 128, 128, vp, vp.shape[1], 0)
    kp_ref = O.quantize_pack_outer(ofmt, kps)
    vp_ref = O.quantize_pack_outer(ofmt, vps)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), kp_ref) and np.array_equal(vp.cpu().numpy(), vp_ref)
    from gpu_common import gpu_decode
    S_ = bench_splits(wl)
    out, _, _ = gpu_decode(fmt, dev(x.q), wl.Hkv, kp, vp, wl.n_packed, dev(kr), dev(vr), wl.n_res,
                           S_, sm=SM, entry=K.kvq_decode_attention_outer)
    torch.cuda.synchronize()
    ref = O.attention_outer(ofmt, x.q, wl.Hkv, kp_ref, vp_ref, wl.n_packed, kr, vr, wl.n_res, sm=SM)
    assert_close(out.cpu().numpy(), ref, "outer attention 32K")
