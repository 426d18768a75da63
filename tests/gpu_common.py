"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and call the
HIP path through the C ABI binding (no computation here)."""
from __future__ import annotations

import os

import numpy as np
import torch

from bit_kv_cache_pack_amd import kvq as K

DEV = "cuda:0"
TOL_MAX_ABS = 2e-3      # attention parity bar (max |gpu - oracle|)
TOL_REL_L2 = 1e-3       # ||gpu - oracle||_2 / ||oracle||_2


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_quantize(fmt: K.Format, src16: np.ndarray, cap_blocks: int | None = None,
                 first_block: int = 0, dst: torch.Tensor | None = None) -> torch.Tensor:
    src = dev(src16)
    rows, T, d = src.shape
    bb = fmt.block_bytes
    if dst is None:
        cap = cap_blocks if cap_blocks is not None else first_block + T // 128
        dst = torch.zeros((rows, cap * bb), dtype=torch.uint8, device=DEV)
    K.kvq_quantize_pack(fmt, src, rows, T, T * d, d, dst, dst.shape[1], first_block)
    return dst


def gpu_decode(fmt: K.Format, q: torch.Tensor, Hkv: int, kp, vp, n_packed: int, kr, vr,
               n_res: int, S: int, out_dtype: int = K.KVQ_OUT_F32, sm: float | None = None,
               entry=None):
    """Decode partials through `entry` (default kvq_decode_attention), then kvq_combine."""
    entry = K.kvq_decode_attention if entry is None else entry
    B, Hq, d = q.shape
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    part_o = torch.empty((B, Hq, S, d), dtype=torch.float32, device=DEV)
    part_lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    stride = kp.shape[1] if kp is not None else 0
    cap = kr.shape[2] if kr is not None else 0
    entry(fmt, q, B, Hq, Hkv, kp, vp, stride, n_packed, kr, vr, cap, n_res, sm, S, part_o,
          part_lse)
    out = torch.empty((B, Hq, d), dtype=torch.float16 if out_dtype == K.KVQ_OUT_F16
                      else torch.float32, device=DEV)
    K.kvq_combine(part_o, part_lse, B, Hq, d, S, out, out_dtype)
    return out, part_o, part_lse


def errors(got, ref) -> tuple[float, float]:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    return float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what=""):
    ma, rl = errors(got, ref)
    if os.environ.get("KVQ_REPORT_ERRORS"):
        print(f"[errors] {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= TOL_MAX_ABS and rl <= TOL_REL_L2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl


def bench_splits(wl) -> int:
    """The split count the benchmark uses for a workload (256 CUs on MI355X)."""
    return K.suggest_splits(wl.B, wl.Hkv, wl.L, 256)
