"""GPU parity of kvq_decode_attention_fp16 (the FP16 flash-decoding baseline) + kvq_combine
against the fp64 CPU oracle's attention over the same fp16 K/V (all tokens unquantized),
with the attention bar of the packed path."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _run(oracle_mod, B, Hq, Hkv, L, S_, stride=None, seed=0, scale=1.0):
    from gpu_common import DEV, assert_close, dev
    O = oracle_mod
    rng = np.random.default_rng(seed)
    stride = L + (L & 1) if stride is None else stride
    k = np.zeros((B, Hkv, stride, 128), np.float16)
    v = np.zeros_like(k)
    k[:, :, :L] = (rng.standard_normal((B, Hkv, L, 128)) * scale).astype(np.float16)
    v[:, :, :L] = (rng.standard_normal((B, Hkv, L, 128)) * scale).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    print(f"[fp16 baseline] B={B} Hq={Hq} Hkv={Hkv} L={L} stride={stride} S={S_} seed={seed}",
          flush=True)
    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_fp16(dev(q), B, Hq, Hkv, dev(k), dev(v), stride, L, SM, S_, po, pl)
    K.kvq_combine(po, pl, B, Hq, 128, S_, out)
    torch.cuda.synchronize()
    empty = np.zeros((B * Hkv, 0), np.uint8)
    ref = O.attention(O.Format(4), q, Hkv, empty, empty, 0, k, v, L, sm=SM)
    return assert_close(out.cpu().numpy(), ref, "fp16 baseline")


@pytest.mark.parametrize("B,Hq,Hkv,L,S_", [
    (1, 8, 2, 1024, 4),
    (1, 8, 2, 1, 1),        # one token
    (1, 8, 2, 33, 3),       # ragged tail, empty splits
    (2, 4, 4, 100, 2),      # gq 1
    (1, 6, 2, 777, 5),      # gq 3 (tail launch only)
    (1, 20, 2, 300, 3),     # gq 10 (chunks + tail)
    (1, 32, 2, 2048, 16),   # gq 16
    (3, 32, 8, 4096, 8),
    (1, 8, 2, 32768, 1024),  # the split limit: one 32-token tile per split
])
def test_fp16_baseline_small(oracle_mod, B, Hq, Hkv, L, S_):
    _run(oracle_mod, B, Hq, Hkv, L, S_, seed=B + Hq + L + S_)


def test_fp16_baseline_row_stride_and_scale(oracle_mod):
    _run(oracle_mod, 1, 8, 2, 500, 3, stride=640, seed=3, scale=4.0)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_fp16_baseline_full_32k(oracle_mod):
    """The llama8b_32k shape with every token in fp16 (the workload's own K, V, q)."""
    from gpu_common import DEV, assert_close, dev
    O = oracle_mod
    wl = S.WORKLOADS["llama8b_32k"]
    x = S.make_inputs(wl)
    S_ = 32
    po = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=DEV)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=DEV)
    print("[fp16 baseline full] decode", flush=True)
    K.kvq_decode_attention_fp16(dev(x.q), wl.B, wl.Hq, wl.Hkv, dev(x.k), dev(x.v), wl.L, wl.L,
                                SM, S_, po, pl)
    K.kvq_combine(po, pl, wl.B, wl.Hq, 128, S_, out)
    torch.cuda.synchronize()
    print("[fp16 baseline full] oracle", flush=True)
    empty = np.zeros((wl.B * wl.Hkv, 0), np.uint8)
    ref = O.attention(O.Format(4), x.q, wl.Hkv, empty, empty, 0, x.k, x.v, wl.L, sm=SM)
    ma, rl = assert_close(out.cpu().numpy(), ref, "fp16 baseline 32K")
    print(f"[fp16 baseline full] max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
