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
