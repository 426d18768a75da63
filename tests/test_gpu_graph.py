"""The decode step (kvq_decode_attention + kvq_combine) captured in a HIP graph and replayed:
every replay, with eager work and synchronizations in between, must give exactly the
output of the eager calls (the benchmark times its steps this way)."""
import math

import numpy as np
import pytest
import torch

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    from gpu_common import DEV, dev, gpu_quantize
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    fmt = K.Format(wl.bits)
    kps, vps = x.packed_src()
    kp = gpu_quantize(fmt, np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128)))
    vp = gpu_quantize(fmt, np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128)))
    kr, vr = (dev(a) for a in x.residual())
    q = dev(x.q)
    S_ = 4
    sm = float(np.float32(1.0 / math.sqrt(128)))
    po = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=DEV)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device=DEV)

    def step(sp):
        K.kvq_decode_attention(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, kp.shape[1], wl.n_packed, kr,
                               vr, 128, wl.n_res, sm, S_, po, pl, stream=sp)
        K.kvq_combine(po, pl, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    print("[graph] eager reference", flush=True)
    step(None)
    torch.cuda.synchronize()
    ref_out, ref_po, ref_pl = out.clone(), po.clone(), pl.clone()

    print("[graph] capture", flush=True)
    side = torch.cuda.Stream(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream(DEV).cuda_stream)
    for rep in range(4):
        out.fill_(0)
        po.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: output differs"
        assert torch.equal(po, ref_po) and torch.equal(pl, ref_pl), f"replay {rep}: partials differ"
        step(None)                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)


def test_fused_append_step_graph_replays_match_eager():
    """kvq_decode_attention_append + kvq_combine captured once; before each replay a new
    token is copied into the staging buffers the graph reads. Every replay's output and the
    window afterwards equal the same calls run eagerly on a copy of the cache."""
    from gpu_common import DEV, dev, gpu_quantize
    wl = S.WORKLOADS["tiny"]
    x = S.make_inputs(wl)
    rows = wl.B * wl.Hkv
    fmt = K.Format(wl.bits)
    kps, vps = x.packed_src()
    kp = gpu_quantize(fmt, np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128)))
    vp = gpu_quantize(fmt, np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128)))
    kr0, vr0 = x.residual()
    krg, vrg, kre, vre = dev(kr0), dev(vr0), dev(kr0), dev(vr0)
    q = dev(x.q)
    S_, n_res = 4, wl.n_res
    sm = float(np.float32(1.0 / math.sqrt(128)))
    kn = torch.zeros((wl.B, wl.Hkv, 128), dtype=torch.float16, device=DEV)
    vn = torch.zeros_like(kn)
    po = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=DEV)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device=DEV)
    poe, ple, oute = torch.empty_like(po), torch.empty_like(pl), torch.empty_like(out)

    def step(kr, vr, po_, pl_, out_, sp):
        K.kvq_decode_attention_append(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, kp.shape[1],
                                      wl.n_packed, kr, vr, 128, n_res, kn, vn, sm, S_, po_, pl_,
                                      stream=sp)
        K.kvq_combine(po_, pl_, wl.B, wl.Hq, 128, S_, out_, K.KVQ_OUT_F16, stream=sp)

    print("[graph fused append] capture", flush=True)
    side = torch.cuda.Stream(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(krg, vrg, po, pl, out, torch.cuda.current_stream(DEV).cuda_stream)
    rng = np.random.default_rng(9)
    for rep in range(5):
        kn.copy_(dev(rng.standard_normal((wl.B, wl.Hkv, 128)).astype(np.float16)))
        vn.copy_(dev(rng.standard_normal((wl.B, wl.Hkv, 128)).astype(np.float16)))
        out.fill_(0)
        torch.cuda.synchronize()
        print(f"[graph fused append] replay {rep}", flush=True)
        g.replay()
        step(kre, vre, poe, ple, oute, None)          # the same step, eagerly, on the copy
        torch.cuda.synchronize()
        assert torch.equal(out, oute), f"replay {rep}: output differs"
        assert torch.equal(po, poe) and torch.equal(pl, ple), f"replay {rep}: partials differ"
        assert torch.equal(krg, kre) and torch.equal(vrg, vre), f"replay {rep}: window differs"
        assert torch.equal(krg[:, :, n_res - 1], kn), f"replay {rep}: new token not stored"


def test_paged_step_graph_replays_match_eager():
    """One paged serving step (kvq_append_evict + kvq_decode_attention_paged + kvq_combine)
    captured once and replayed for 40 steps, the new tokens and q copied in before each
    replay: every step's output, and the pools, windows and sequence states at the end,
    equal those of the same 40 steps run eagerly on a copy."""
    from gpu_common import DEV, dev
    import paged_common as P
    rng = np.random.default_rng(5)
    fmt = K.Format(4)
    B, Hq, Hkv, cap, n_sink, S_, steps = 3, 8, 2, 16, 2, 3, 40
    n_packed = [100, 0, 300]
    n_res = [cap, 5, cap]
    tbl, npool = P.make_table(rng, B, [P.blocks_for(n + steps + 1) for n in n_packed])
    bb = fmt.block_bytes
    kpool0 = dev(rng.integers(0, 256, (npool, Hkv, bb), dtype=np.uint8))
    vpool0 = dev(rng.integers(0, 256, (npool, Hkv, bb), dtype=np.uint8))
    # keep the packed bytes' scale/zero finite: pack real tokens into every used position
    zero = torch.zeros(B, dtype=torch.int32, device=DEV)
    cnt = dev(np.array(n_packed, np.int32))
    src = dev(np.asarray(rng.standard_normal((B * Hkv, 300, 128)), np.float16))
    dtbl = dev(tbl)
    K.kvq_pack_tokens_paged(fmt, src, B, Hkv, 300 * 128, 128, cnt, zero, 300, kpool0, npool,
                            Hkv * bb, bb, dtbl, tbl.shape[1])
    K.kvq_pack_tokens_paged(fmt, src, B, Hkv, 300 * 128, 128, cnt, zero, 300, vpool0, npool,
                            Hkv * bb, bb, dtbl, tbl.shape[1])
    kres0 = dev(np.asarray(rng.standard_normal((B, Hkv, cap, 128)), np.float16))
    vres0 = dev(np.asarray(rng.standard_normal((B, Hkv, cap, 128)), np.float16))
    st0 = dev(np.array([[n_packed[b], n_res[b], n_sink, 0] for b in range(B)], np.int32))
    new_k = dev(np.asarray(rng.standard_normal((steps, B, Hkv, 128)), np.float16))
    new_v = dev(np.asarray(rng.standard_normal((steps, B, Hkv, 128)), np.float16))
    qs = dev(np.asarray(rng.standard_normal((steps, B, Hq, 128)), np.float16))
    sm = float(np.float32(1.0 / math.sqrt(128)))

    def make():
        return [t.clone() for t in (kpool0, vpool0, kres0, vres0, st0)]

    def step(bufs, kn, vn, q, po, pl, out, sp):
        kp, vp, kr, vr, st = bufs
        K.kvq_append_evict(fmt, kn, vn, kr, vr, cap, n_sink, kp, vp, npool, Hkv * bb, bb, dtbl,
                           tbl.shape[1], st, B, Hkv, stream=sp)
        K.kvq_decode_attention_paged(fmt, q, B, Hq, Hkv, kp, vp, npool, Hkv * bb, bb, dtbl,
                                     tbl.shape[1], st, kr, vr, cap, sm, S_, po, pl, stream=sp)
        K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F32, stream=sp)

    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    print("[graph paged] eager", flush=True)
    eager = make()
    ref_out = []
    for i in range(steps):
        step(eager, new_k[i], new_v[i], qs[i], po, pl, out, None)
        ref_out.append(out.clone())
    torch.cuda.synchronize()

    print("[graph paged] capture + replays", flush=True)
    g_bufs = make()
    kn_in, vn_in, q_in = new_k[0].clone(), new_v[0].clone(), qs[0].clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV)
    g = torch.cuda.CUDAGraph()
    # capture on a copy of the buffers, so that capturing does not advance the real ones
    cap_bufs = make()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step(cap_bufs, kn_in, vn_in, q_in, po, pl, out, torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    # the graph reads and writes cap_bufs: reset them to the initial state, then replay
    for dst, srcb in zip(cap_bufs, g_bufs):
        dst.copy_(srcb)
    torch.cuda.synchronize()
    for i in range(steps):
        kn_in.copy_(new_k[i])
        vn_in.copy_(new_v[i])
        q_in.copy_(qs[i])
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out[i]), f"step {i}: output differs"
    for a, b_, name in zip(cap_bufs, eager, ("K pool", "V pool", "K window", "V window", "state")):
        assert torch.equal(a, b_), name
