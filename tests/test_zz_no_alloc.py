"""GPU check of the allocation-free fused decode (kvq_decode_attention_fused_noalloc): called
through the C ABI, its output equals kvq_decode_attention_fused's (same kernels, records in the
library's scratch array instead of a caller workspace) on two calls in a row, the second with
a smaller input, and matches the fp64 oracle within the attention bar."""
import numpy as np
import pytest
import torch

from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _case(O, rng, bits, B, Hq, Hkv, n_packed, n_res, cap=128):
    from gpu_common import dev, gpu_quantize
    rows = B * Hkv
    fmt, ofmt = K.Format(bits), O.Format(bits)
    ks = _f16(rng.standard_normal((rows, n_packed, 128)))
    vs = _f16(rng.standard_normal((rows, n_packed, 128)))
    kr = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vr = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    kp, vp = gpu_quantize(fmt, ks), gpu_quantize(fmt, vs)
    kpr, vpr = O.quantize_pack(ofmt, ks), O.quantize_pack(ofmt, vs)
    ref = O.attention(ofmt, q, Hkv, kpr, vpr, n_packed, kr, vr, n_res, sm=SM)
    return dict(fmt=fmt, q=dev(q), kp=kp, vp=vp, kr=dev(kr), vr=dev(vr), ref=ref, B=B, Hq=Hq,
                Hkv=Hkv, n_packed=n_packed, n_res=n_res, cap=cap)


def _both(c, S_):
    from gpu_common import DEV
    B, Hq, Hkv = c["B"], c["Hq"], c["Hkv"]
    args = (c["fmt"], c["q"], B, Hq, Hkv, c["kp"], c["vp"], c["kp"].shape[1], c["n_packed"],
            c["kr"], c["vr"], c["cap"], c["n_res"], SM, S_)
    a = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full_like(a, float("nan"))
    K.kvq_decode_attention_fused_noalloc(*args, a, K.KVQ_OUT_F32)
    nws = K.kvq_decode_workspace_bytes(B, Hq, Hkv, S_)
    ws = torch.zeros(max(nws, 256), dtype=torch.uint8, device=DEV)
    K.kvq_decode_attention_fused(*args, ws, ws.numel(), b, K.KVQ_OUT_F32)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_equals_workspace_call_twice_then_smaller(oracle_mod):
    from gpu_common import assert_close
    O = oracle_mod
    rng = np.random.default_rng(77)
    print("[noalloc] call 1: B=2 Hq=16 Hkv=4 4096 packed + 100 window, S=64", flush=True)
    big = _case(O, rng, 4, 2, 16, 4, 4096, 100)
    a, b = _both(big, 64)
    assert torch.equal(a, b), "call 1 differs from the workspace call"
    assert_close(a.cpu().numpy(), big["ref"], "noalloc call 1")
    print("[noalloc] call 2: B=1 Hq=8 Hkv=2 1024 packed + 17 window, S=9", flush=True)
    small = _case(O, rng, 3, 1, 8, 2, 1024, 17)
    a2, b2 = _both(small, 9)
    assert torch.equal(a2, b2), "call 2 differs from the workspace call"
    assert_close(a2.cpu().numpy(), small["ref"], "noalloc call 2")
    print("[noalloc] call 3: the first shape again", flush=True)
    a3, _ = _both(big, 64)
    assert torch.equal(a3, a)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """8 rows of 4 query heads at 1024 splits need 17.6 MB of records: rejected on the host
    with KVQ_ERR_TOO_LARGE before anything is launched."""
    from gpu_common import DEV
    fmt = K.Format(4)
    q = torch.zeros((1, 32, 128), dtype=torch.float16, device=DEV)
    kp = torch.zeros((8, 256 * fmt.block_bytes), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=DEV)
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 1024) > K.KVQ_NOALLOC_SCRATCH_BYTES
    with pytest.raises(K.KVQError) as e:
        K.kvq_decode_attention_fused_noalloc(fmt, q, 1, 32, 8, kp, kp, kp.shape[1], 32768, None,
                                             None, 0, 0, SM, 1024, out)
    assert e.value.status == K.KVQ_ERR_TOO_LARGE
