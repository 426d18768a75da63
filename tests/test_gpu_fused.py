"""GPU parity of the fused decode step (kvq_decode_attention_fused and
kvq_decode_attention_paged_fused: the split-K partials merged into the output inside the
decode launch) against the fp64 CPU oracle.

Bar: max |gpu - oracle| <= 2e-3 and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3 over the
whole output, as for kvq_decode_attention + kvq_combine. The output buffer starts as NaN,
so a (b, h) that no workgroup writes fails; every test also calls twice on one workspace
(the second call only works if the first left every counter at zero) and expects the same
bits, since the merge order does not depend on which workgroup arrives last."""
import numpy as np
import pytest
import torch

import paged_common as P
import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K
from test_gpu_decode import APPEND_CASES, CASES, SM, _case, _f16, _random_cases

pytestmark = pytest.mark.gpu


def _workspace(B, Hq, Hkv, S_, extra=0):
    from gpu_common import DEV
    n = K.kvq_decode_workspace_bytes(B, Hq, Hkv, S_)
    return torch.zeros(max(n + extra, 256), dtype=torch.uint8, device=DEV)


def gpu_fused(fmt, q, Hkv, kp, vp, n_packed, kr, vr, n_res, S_, ws=None,
              out_dtype=K.KVQ_OUT_F32, key_norm=None, k_new=None, v_new=None):
    from gpu_common import DEV
    B, Hq, d = q.shape
    if ws is None:
        ws = _workspace(B, Hq, Hkv, S_)
    stride = kp.shape[1] if kp is not None else 0
    cap = kr.shape[2] if kr is not None else 0
    out = torch.full((B, Hq, d), float("nan"), device=DEV,
                     dtype=torch.float16 if out_dtype == K.KVQ_OUT_F16 else torch.float32)
    K.kvq_decode_attention_fused(fmt, q, B, Hq, Hkv, kp, vp, stride, n_packed, kr, vr, cap, n_res,
                                 SM, S_, ws, ws.numel(), out, out_dtype, key_norm=key_norm,
                                 k_new_fp16=k_new, v_new_fp16=v_new)
    return out


def _inputs(O, bits, hybrid, B, Hq, Hkv, n_packed, n_res, seed, cap=128, dist="normal",
            scale=1.0):
    from gpu_common import dev, gpu_quantize
    rng = np.random.default_rng(seed)
    q, ksrc, vsrc, kr, vr = _case(rng, B, Hq, Hkv, n_packed, n_res, dist, scale, cap)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    rows = B * Hkv
    if n_packed:
        kp_ref = O.quantize_pack(ofmt, ksrc.reshape(rows, n_packed, 128))
        vp_ref = O.quantize_pack(ofmt, vsrc.reshape(rows, n_packed, 128))
        kp = gpu_quantize(fmt, ksrc.reshape(rows, n_packed, 128))
        vp = gpu_quantize(fmt, vsrc.reshape(rows, n_packed, 128))
        assert np.array_equal(kp.cpu().numpy(), kp_ref)
        assert np.array_equal(vp.cpu().numpy(), vp_ref)
    else:
        kp_ref = vp_ref = np.zeros((rows, 0), np.uint8)
        kp = vp = None
    ref = O.attention(ofmt, q, Hkv, kp_ref, vp_ref, n_packed, kr, vr, n_res, sm=SM)
    return dict(fmt=fmt, q=dev(q), kp=kp, vp=vp, kr=dev(kr), vr=dev(vr), ref=ref)


def _check(O, bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_, seed, cap=128, dist="normal",
           scale=1.0):
    from gpu_common import assert_close
    print(f"[fused] bits={bits} hybrid={hybrid} B={B} Hq={Hq} Hkv={Hkv} n_packed={n_packed} "
          f"n_res={n_res} S={S_} seed={seed}", flush=True)
    c = _inputs(O, bits, hybrid, B, Hq, Hkv, n_packed, n_res, seed, cap, dist, scale)
    ws = _workspace(B, Hq, Hkv, S_)
    args = (c["fmt"], c["q"], Hkv, c["kp"], c["vp"], n_packed, c["kr"], c["vr"], n_res, S_)
    a = gpu_fused(*args, ws=ws)
    b = gpu_fused(*args, ws=ws)
    h = gpu_fused(*args, ws=ws, out_dtype=K.KVQ_OUT_F16)
    torch.cuda.synchronize()
    got = a.cpu().numpy()
    assert torch.equal(a, b), "a second call on the same workspace differs"
    # the fp16 output is the round-to-nearest-even of the fp32 value
    assert np.array_equal(h.cpu().numpy(), got.astype(np.float16))
    return assert_close(got, c["ref"], "fused attention")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}h{}_B{}_{}x{}_P{}_R{}_S{}".format(*c))
def test_fused_small(oracle_mod, case):
    bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_ = case
    _check(oracle_mod, bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_, seed=sum(case))


@pytest.mark.parametrize("S_", [2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 511, 512, 513, 993,
                                1023, 1024])
def test_fused_split_tree_shapes(oracle_mod, S_):
    """Split counts that fill the fan-in-32 tree exactly (32, 1024), leave a lone child at the
    first level (33, 65, 513, 993), or give one or two levels, over 32K packed tokens (1024
    tiles) and a full window."""
    _check(oracle_mod, 4, False, 1, 8, 2, 32768, 128, S_, seed=40 + S_)


@pytest.mark.parametrize("dist,scale", [("t5", 1.0), ("normal", 4.0), ("normal", 0.05)])
def test_fused_value_ranges(oracle_mod, dist, scale):
    _check(oracle_mod, 4, False, 1, 8, 2, 640, 128, 5, seed=7, dist=dist, scale=scale)
    _check(oracle_mod, 2, True, 1, 8, 2, 640, 128, 5, seed=8, dist=dist, scale=scale)


@pytest.mark.parametrize("case", _random_cases(24, seed=4048), ids=lambda c: f"r{c[0]}")
def test_fused_random_shapes(oracle_mod, case):
    i, bits, hybrid, B, Hq, Hkv, n_packed, n_res, cap, S_ = case
    _check(oracle_mod, bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_, seed=900 + i, cap=cap)


def test_fused_workspace_shared_by_different_shapes(oracle_mod):
    """One zeroed workspace, large enough for the largest call, used by calls of different
    shapes and split counts in turn: each call leaves it ready for the next."""
    from gpu_common import assert_close
    O = oracle_mod
    shapes = [(4, False, 2, 16, 4, 2048, 100, 64), (3, False, 1, 12, 4, 1024, 5, 9),
              (2, True, 3, 8, 2, 512, 128, 513), (4, False, 2, 16, 4, 2048, 100, 64)]
    ws = _workspace(3, 16, 4, 1024)
    first = None
    for k, (bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_) in enumerate(shapes):
        print(f"[fused shared workspace] call {k}: S={S_}", flush=True)
        c = _inputs(O, bits, hybrid, B, Hq, Hkv, n_packed, n_res, seed=60 + (k % 3))
        out = gpu_fused(c["fmt"], c["q"], Hkv, c["kp"], c["vp"], n_packed, c["kr"], c["vr"],
                        n_res, S_, ws=ws)
        assert_close(out.cpu().numpy(), c["ref"], f"call {k}")
        if k == 0:
            first = out.clone()
        if k == 3:
            assert torch.equal(out, first)


@pytest.mark.parametrize("case", APPEND_CASES,
                         ids=lambda c: "b{}h{}_B{}_{}x{}_P{}_C{}_R{}_S{}".format(*c))
def test_fused_append(oracle_mod, case):
    """The new token of every row enters window slot n_res - 1 inside the fused launch: the
    window afterwards equals kvq_append_residual's, and the output matches the oracle on
    the updated cache."""
    from gpu_common import assert_close, dev, gpu_quantize
    O = oracle_mod
    bits, hybrid, B, Hq, Hkv, n_packed, cap, n_res, S_ = case
    rng = np.random.default_rng(700 + sum(case))
    rows = B * Hkv
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    q = _f16(rng.standard_normal((B, Hq, 128)))
    kr = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    kn = _f16(rng.standard_normal((B, Hkv, 128)) * 2)
    vn = _f16(rng.standard_normal((B, Hkv, 128)) * 2)
    print(f"[fused append] case={case}", flush=True)
    if n_packed:
        ks = _f16(rng.standard_normal((rows, n_packed, 128)))
        vs = _f16(rng.standard_normal((rows, n_packed, 128)))
        kp, vp = gpu_quantize(fmt, ks), gpu_quantize(fmt, vs)
        kpr, vpr = O.quantize_pack(ofmt, ks), O.quantize_pack(ofmt, vs)
    else:
        kp = vp = None
        kpr = vpr = np.zeros((rows, 0), np.uint8)
    qd, knd, vnd = dev(q), dev(kn), dev(vn)
    kra, vra, krb, vrb = dev(kr), dev(vr), dev(kr), dev(vr)
    K.kvq_append_residual(knd, vnd, kra, vra, B, Hkv, 128, cap, n_res - 1)
    out = gpu_fused(fmt, qd, Hkv, kp, vp, n_packed, krb, vrb, n_res, S_, k_new=knd, v_new=vnd)
    torch.cuda.synchronize()
    assert torch.equal(kra, krb) and torch.equal(vra, vrb), "windows differ"
    kr2, vr2 = kr.copy(), vr.copy()
    kr2[:, :, n_res - 1], vr2[:, :, n_res - 1] = kn, vn
    ref = O.attention(ofmt, q, Hkv, kpr, vpr, n_packed, kr2, vr2, n_res, sm=SM)
    assert_close(out.cpu().numpy(), ref, "fused attention after append")


@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, False), (2, True)])
def test_fused_normalized_pipeline(oracle_mod, bits, hybrid):
    """Key-channel normalization with the fused decode: factors, scaled keys and window on
    the GPU, q multiplied inside the fused launch; against the same steps in the oracle."""
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
    print(f"[fused knorm pipeline] bits={bits} hybrid={hybrid}", flush=True)
    n_ref = O.key_norm(kps)
    kn_ref = O.channel_scale(kps, n_ref).view(np.float16)
    krn_ref = O.channel_scale(kr.reshape(rows, -1, 128), n_ref).view(np.float16).reshape(kr.shape)
    qn_ref = O.channel_scale(x.q.reshape(wl.B * wl.Hq, 1, 128), n_ref, rows_per_norm=wl.gq,
                             multiply=True).view(np.float16).reshape(x.q.shape)
    kp_ref = O.quantize_pack(ofmt, kn_ref)
    vp_ref = O.quantize_pack(ofmt, vps)
    ref = O.attention(ofmt, qn_ref, wl.Hkv, kp_ref, vp_ref, wl.n_packed, krn_ref, vr, wl.n_res,
                      sm=SM)
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
    out = gpu_fused(fmt, dev(x.q), wl.Hkv, kp, vp, wl.n_packed, krd, dev(vr), wl.n_res, 4,
                    key_norm=nd)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), kp_ref)
    assert_close(out.cpu().numpy(), ref, "fused normalized attention")


# ---------------------------------------------------------------- paged cache ----

def _paged(O, bits, hybrid, B, Hq, Hkv, n_packed, n_res, cap, seed):
    from gpu_common import dev
    from test_gpu_paged import _paged_case
    rng = np.random.default_rng(seed)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    c = _paged_case(O, rng, fmt, ofmt, B, Hq, Hkv, n_packed, n_res, cap)
    ref = O.attention_paged(ofmt, c["q"], Hkv, c["kpool"], c["vpool"], c["tbl"], c["state"],
                            c["kres"], c["vres"], sm=SM, block_stride=c["bs"],
                            head_stride=c["hs"])
    d = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    return fmt, c, d, ref


def _gpu_paged_fused(fmt, c, d, B, Hq, Hkv, S_, ws):
    from gpu_common import DEV
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_paged_fused(fmt, d["q"], B, Hq, Hkv, d["kpool"], d["vpool"],
                                       c["npool"], c["bs"], c["hs"], d["tbl"], c["tbl"].shape[1],
                                       d["state"], d["kres"], d["vres"], c["cap"], SM, S_, ws,
                                       ws.numel(), out, K.KVQ_OUT_F32)
    return out


PAGED_CASES = [
    # bits, hybrid, B, Hq, Hkv, n_packed per sequence, n_res per sequence, cap, S
    (4, False, 4, 8, 2, [300, 1, 31, 1000], [10, 0, 128, 5], 128, 3),
    (4, False, 3, 32, 8, [33, 4096, 0], [0, 17, 40], 64, 5),
    (3, True, 2, 6, 1, [517, 64], [3, 3], 16, 2),
    (2, False, 5, 16, 16, [1, 2, 127, 128, 129], [1, 0, 0, 7, 2], 8, 1),
    (4, False, 2, 20, 2, [640, 333], [16, 16], 16, 4),
    (4, False, 2, 8, 2, [32768, 700], [128, 3], 128, 1024),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"b{c[0]}_B{c[2]}_S{c[8]}")
def test_paged_fused_matches_oracle(oracle_mod, case):
    from gpu_common import assert_close
    bits, hybrid, B, Hq, Hkv, n_packed, n_res, cap, S_ = case
    print(f"[paged fused] {case}", flush=True)
    fmt, c, d, ref = _paged(oracle_mod, bits, hybrid, B, Hq, Hkv, n_packed, n_res, cap,
                            seed=sum(n_packed) + bits)
    ws = _workspace(B, Hq, Hkv, S_)
    a = _gpu_paged_fused(fmt, c, d, B, Hq, Hkv, S_, ws)
    b = _gpu_paged_fused(fmt, c, d, B, Hq, Hkv, S_, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert_close(a.cpu().numpy(), ref, "paged fused attention")


def test_paged_fused_empty_sequence_gives_zero(oracle_mod):
    """A sequence with no packed token and an empty window (a fresh slot of a ragged batch)
    attends nothing: its output is 0, with the fused merge and with kvq_combine alike."""
    from gpu_common import DEV, assert_close
    B, Hq, Hkv, S_ = 3, 8, 2, 4
    fmt, c, d, ref = _paged(oracle_mod, 4, False, B, Hq, Hkv, [500, 0, 64], [3, 0, 0], 16, seed=5)
    print("[paged fused] empty sequence", flush=True)
    ws = _workspace(B, Hq, Hkv, S_)
    out = _gpu_paged_fused(fmt, c, d, B, Hq, Hkv, S_, ws).cpu().numpy()
    assert np.all(out[1] == 0)
    assert_close(out[[0, 2]], ref[[0, 2]], "paged fused attention, non-empty sequences")
    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_paged(fmt, d["q"], B, Hq, Hkv, d["kpool"], d["vpool"], c["npool"],
                                 c["bs"], c["hs"], d["tbl"], c["tbl"].shape[1], d["state"],
                                 d["kres"], d["vres"], c["cap"], SM, S_, po, pl)
    o2 = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_combine(po, pl, B, Hq, 128, S_, o2, K.KVQ_OUT_F32)
    o2 = o2.cpu().numpy()
    assert np.all(o2[1] == 0)
    assert_close(o2[[0, 2]], ref[[0, 2]], "paged + combine, non-empty sequences")


# ------------------------------------------------------------------ full workloads ----

@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "batch8_2bit_hybrid", "long_128k_3bit",
                                  "mha_b64_append"])
def test_fused_full_workload(oracle_mod, name):
    """Every workload at full size with the split count the benchmark uses (one split, so
    no merge, at the MHA workload): every output against the oracle."""
    from gpu_common import assert_close, bench_splits, dev, gpu_quantize
    O = oracle_mod
    wl = S.WORKLOADS[name]
    print(f"[fused full] {name}: inputs", flush=True)
    x = S.make_inputs(wl)
    kps, vps = x.packed_src()
    kr, vr = x.residual()
    fmt, ofmt = K.Format(wl.bits, 128, wl.hybrid), O.Format(wl.bits, 128, wl.hybrid)
    rows = wl.B * wl.Hkv
    kps = np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))
    vps = np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))
    kp, vp = gpu_quantize(fmt, kps), gpu_quantize(fmt, vps)
    S_ = bench_splits(wl)
    print(f"[fused full] {name}: S={S_}", flush=True)
    out = gpu_fused(fmt, dev(x.q), wl.Hkv, kp, vp, wl.n_packed, dev(kr), dev(vr), wl.n_res, S_)
    got = out.cpu().numpy()
    del kp, vp
    print(f"[fused full] {name}: oracle", flush=True)
    kp_ref, vp_ref = O.quantize_pack(ofmt, kps), O.quantize_pack(ofmt, vps)
    ref = O.attention(ofmt, x.q, wl.Hkv, kp_ref, vp_ref, wl.n_packed, kr, vr, wl.n_res, sm=SM)
    ma, rl = assert_close(got, ref, name)
    print(f"[fused full] {name}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)


@pytest.mark.slow
def test_paged_fused_full_size_ragged(oracle_mod):
    from gpu_common import assert_close
    from test_gpu_paged import _paged_from_inputs
    O = oracle_mod
    wl = S.PAGED_WORKLOADS["paged_ragged_b16"]
    x = S.make_paged_inputs(wl)
    fmt, ofmt = K.Format(wl.bits), O.Format(wl.bits)
    print(f"[paged fused] full size {wl.name}", flush=True)
    c = _paged_from_inputs(O, ofmt, wl, x)
    from gpu_common import dev
    d = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    S_ = K.suggest_splits_paged(int(x.n_packed.sum()), int(x.n_packed.max()), wl.Hkv, 256)
    out = _gpu_paged_fused(fmt, c, d, wl.B, wl.Hq, wl.Hkv, S_, _workspace(wl.B, wl.Hq, wl.Hkv, S_))
    ref = O.attention_paged(ofmt, c["q"], wl.Hkv, c["kpool"], c["vpool"], c["tbl"], c["state"],
                            c["kres"], c["vres"], sm=SM, block_stride=c["bs"], head_stride=c["hs"])
    assert_close(out.cpu().numpy(), ref, "full-size paged fused attention")
