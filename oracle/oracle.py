"""numpy front end of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
It loads liboracle.so (built from kvq_oracle.c by build_oracle.py) and passes numpy
arrays to it; every number it returns is computed by the C oracle. fp16 data travels as
uint16 bit patterns, packed caches as uint8 arrays.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_ORACLE_LIB_PATH may name another build of the oracle (the sanitizer-checked one)
_LIB_PATH = os.environ.get("KVQ_ORACLE_LIB_PATH") or os.path.join(HERE, "liboracle.so")
_lib = None

GROUP = 32
BLOCK = 128


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build_oracle
            build_oracle.build()
        _lib = C.CDLL(_LIB_PATH)
        _setup(_lib)
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _setup(L):
    i32, i64, f32, f64, vp = C.c_int, C.c_int64, C.c_float, C.c_double, C.c_void_p
    L.oq_f16_to_f32.argtypes = [C.c_uint16]
    L.oq_f16_to_f32.restype = f32
    L.oq_f32_to_f16.argtypes = [f32]
    L.oq_f32_to_f16.restype = C.c_uint16
    L.oq_asym_candidate.argtypes = [vp, i32, vp, vp, vp]
    L.oq_sym_candidate.argtypes = [vp, i32, vp, vp, vp]
    L.oq_sym_candidate.restype = i32
    L.oq_group_sse.argtypes = [vp, vp, C.c_uint16, C.c_uint16]
    L.oq_group_sse.restype = f32
    L.oq_quantize_group.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    L.oq_pack_codes.argtypes = [vp, i32, vp]
    L.oq_unpack_codes.argtypes = [vp, i32, vp]
    for n in ("oq_codes_bytes",):
        getattr(L, n).argtypes = [i32, i32]
        getattr(L, n).restype = i64
    L.oq_sz_bytes.argtypes = [i32]
    L.oq_sz_bytes.restype = i64
    L.oq_flag_bytes.argtypes = [i32, i32]
    L.oq_flag_bytes.restype = i64
    L.oq_sz_offset.argtypes = [i32, i32]
    L.oq_sz_offset.restype = i64
    L.oq_flag_offset.argtypes = [i32, i32]
    L.oq_flag_offset.restype = i64
    L.oq_block_bytes.argtypes = [i32, i32, i32]
    L.oq_block_bytes.restype = i64
    L.oq_quantize_pack.argtypes = [i32, i32, i32, vp, i64, i32, i64, i64, vp, i64, i32, i32]
    L.oq_quantize_pack.restype = i32
    L.oq_dequant.argtypes = [i32, i32, i32, vp, i64, i64, i64, vp]
    L.oq_attention.argtypes = [i32, i32, i32, vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, i32,
                               i32, f64, vp, i32]
    L.oq_split_attention.argtypes = [i32, i32, i32, vp, i32, i32, i32, vp, vp, i64, i32, vp, vp,
                                     i32, i32, f64, i32, vp, vp, i32]
    L.oq_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    L.oq_split_range.argtypes = [i32, i32, i32, i32, C.POINTER(i64), C.POINTER(i64)]
    L.oq_key_norm.argtypes = [vp, i64, i64, i64, i64, i32, vp]
    L.oq_channel_scale.argtypes = [vp, i64, i64, i64, i64, i32, vp, i64, i32, vp, i64, i64]
    L.oq_quantize_pack_outer.argtypes = [i32, i32, vp, i64, i32, i64, i64, vp, i64, i32]
    L.oq_quantize_pack_outer.restype = i32
    L.oq_attention_outer.argtypes = L.oq_attention.argtypes[:2] + L.oq_attention.argtypes[3:]
    L.oq_split_attention_outer.argtypes = (L.oq_split_attention.argtypes[:2] +
                                           L.oq_split_attention.argtypes[3:])
    L.oq_pack_tokens_paged.argtypes = [i32, i32, i32, vp, i32, i32, i64, i64, vp, vp, vp, i64,
                                       i64, vp, i32]
    L.oq_append_evict.argtypes = [i32, i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, vp,
                                  i32, vp, i32, i32]
    L.oq_attention_paged.argtypes = [i32, i32, i32, vp, i32, i32, i32, vp, vp, i64, i64, vp,
                                     i32, vp, vp, vp, i32, f64, i32, vp, vp, i32]
    L.oq_paged_split_range.argtypes = [i64, i64, i32, i32, C.POINTER(i64), C.POINTER(i64)]


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------------------------------
# fp16 helpers
# ----------------------------------------------------------------------------------------

def f32_to_f16(x: float) -> int:
    return int(lib().oq_f32_to_f16(C.c_float(x)))


def f16_to_f32(h: int) -> float:
    return float(lib().oq_f16_to_f32(C.c_uint16(h)))


def as_bits(a) -> np.ndarray:
    """fp16 array (or uint16 bit patterns) -> contiguous uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise TypeError(f"expected float16 or uint16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a).view(np.uint16)


# ----------------------------------------------------------------------------------------
# Group level
# ----------------------------------------------------------------------------------------

@dataclass
class GroupResult:
    scale: int       # fp16 bits
    zero: int        # fp16 bits
    codes: np.ndarray
    flag: int = 1    # 1 = asym, 0 = sym


def quantize_group(x16: np.ndarray, bits: int, hybrid: bool = False) -> GroupResult:
    x = as_bits(x16)
    assert x.shape == (GROUP,)
    s, z = C.c_uint16(), C.c_uint16()
    codes = np.zeros(GROUP, np.uint8)
    flag = C.c_int()
    lib().oq_quantize_group(_p(x), bits, int(hybrid), C.byref(s), C.byref(z), _p(codes),
                            C.byref(flag))
    return GroupResult(s.value, z.value, codes, flag.value)


def asym_candidate(x16: np.ndarray, bits: int) -> GroupResult:
    x = as_bits(x16)
    s, z = C.c_uint16(), C.c_uint16()
    codes = np.zeros(GROUP, np.uint8)
    lib().oq_asym_candidate(_p(x), bits, C.byref(s), C.byref(z), _p(codes))
    return GroupResult(s.value, z.value, codes, 1)


def sym_candidate(x16: np.ndarray, bits: int) -> tuple[GroupResult, bool]:
    x = as_bits(x16)
    s, z = C.c_uint16(), C.c_uint16()
    codes = np.zeros(GROUP, np.uint8)
    ok = lib().oq_sym_candidate(_p(x), bits, C.byref(s), C.byref(z), _p(codes))
    return GroupResult(s.value, z.value, codes, 0), bool(ok)


def group_sse(x16: np.ndarray, codes: np.ndarray, scale: int, zero: int) -> float:
    x = as_bits(x16)
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return float(lib().oq_group_sse(_p(x), _p(c), scale, zero))


def pack_codes(codes: np.ndarray, bits: int) -> bytes:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(GROUP * bits // 8, np.uint8)
    lib().oq_pack_codes(_p(c), bits, _p(out))
    return out.tobytes()


def unpack_codes(data: bytes, bits: int) -> np.ndarray:
    buf = np.frombuffer(data, np.uint8).copy()
    codes = np.zeros(GROUP, np.uint8)
    lib().oq_unpack_codes(_p(buf), bits, _p(codes))
    return codes


# ----------------------------------------------------------------------------------------
# Block format
# ----------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Format:
    bits: int
    head_dim: int = 128
    hybrid: bool = False

    @property
    def codes_bytes(self) -> int:
        return int(lib().oq_codes_bytes(self.bits, self.head_dim))

    @property
    def sz_offset(self) -> int:
        return int(lib().oq_sz_offset(self.bits, self.head_dim))

    @property
    def sz_bytes(self) -> int:
        return int(lib().oq_sz_bytes(self.head_dim))

    @property
    def flag_offset(self) -> int:
        return int(lib().oq_flag_offset(self.bits, self.head_dim))

    @property
    def flag_bytes(self) -> int:
        return int(lib().oq_flag_bytes(self.head_dim, int(self.hybrid)))

    @property
    def block_bytes(self) -> int:
        return int(lib().oq_block_bytes(self.bits, self.head_dim, int(self.hybrid)))


def quantize_pack(fmt: Format, src16: np.ndarray, n_tokens: int | None = None,
                  n_blocks_capacity: int | None = None, first_block: int = 0,
                  dst: np.ndarray | None = None, n_threads: int | None = None) -> np.ndarray:
    """src16: fp16 [rows][T][head_dim] (or uint16 bits). Quantizes tokens [0, n_tokens)
    into blocks first_block.. of a packed array [rows][capacity * block_bytes] (uint8)."""
    src = as_bits(src16)
    rows, T, d = src.shape
    assert d == fmt.head_dim
    n_tokens = T if n_tokens is None else n_tokens
    nb = n_tokens // BLOCK
    cap = first_block + nb if n_blocks_capacity is None else n_blocks_capacity
    bb = fmt.block_bytes
    if dst is None:
        dst = np.zeros((rows, cap * bb), np.uint8)
    assert dst.dtype == np.uint8 and dst.flags.c_contiguous and dst.shape[0] == rows
    rc = lib().oq_quantize_pack(fmt.bits, d, int(fmt.hybrid), _p(src), rows, n_tokens, T * d, d,
                                _p(dst), dst.shape[1], first_block,
                                n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the quantize arguments")
    return dst


def dequant(fmt: Format, packed: np.ndarray, n_tokens: int) -> np.ndarray:
    rows = packed.shape[0]
    out = np.zeros((rows, n_tokens, fmt.head_dim), np.float64)
    packed = np.ascontiguousarray(packed)
    lib().oq_dequant(fmt.bits, fmt.head_dim, int(fmt.hybrid), _p(packed), rows, n_tokens,
                     packed.shape[1], _p(out))
    return out


# ----------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------

def _att_args(fmt, q16, Hkv, kp, vp, n_packed, kres16, vres16, n_res):
    q = as_bits(q16)
    B, Hq, d = q.shape
    assert d == fmt.head_dim and Hq % Hkv == 0
    kp = np.ascontiguousarray(kp)
    vp = np.ascontiguousarray(vp)
    assert kp.shape == vp.shape and kp.shape[0] == B * Hkv
    if kres16 is None:
        kres = np.zeros((B, Hkv, 1, d), np.uint16)
        vres = kres
        assert n_res == 0
    else:
        kres, vres = as_bits(kres16), as_bits(vres16)
        assert kres.shape[:2] == (B, Hkv) and kres.shape[3] == d
    res_cap = kres.shape[2]
    assert 0 <= n_res <= res_cap
    return q, B, Hq, d, kp, vp, kres, vres, res_cap


def attention(fmt: Format, q16, Hkv: int, kp, vp, n_packed: int, kres16=None, vres16=None,
              n_res: int = 0, sm: float | None = None, n_threads: int | None = None):
    """fp64 out[B][Hq][d] of softmax(sm q K^T) V over packed + residual tokens."""
    q, B, Hq, d, kp, vp, kres, vres, res_cap = _att_args(fmt, q16, Hkv, kp, vp, n_packed,
                                                         kres16, vres16, n_res)
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    out = np.zeros((B, Hq, d), np.float64)
    lib().oq_attention(fmt.bits, d, int(fmt.hybrid), _p(q), B, Hq, Hkv, _p(kp), _p(vp),
                       kp.shape[1], n_packed, _p(kres), _p(vres), res_cap, n_res, sm, _p(out),
                       n_threads or default_threads())
    return out


def split_attention(fmt: Format, q16, Hkv: int, kp, vp, n_packed: int, kres16=None, vres16=None,
                    n_res: int = 0, S: int = 1, sm: float | None = None,
                    n_threads: int | None = None):
    """fp64 partials: part_o[B][Hq][S][d] (normalised) and part_lse[B][Hq][S]."""
    q, B, Hq, d, kp, vp, kres, vres, res_cap = _att_args(fmt, q16, Hkv, kp, vp, n_packed,
                                                         kres16, vres16, n_res)
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    po = np.zeros((B, Hq, S, d), np.float64)
    pl = np.zeros((B, Hq, S), np.float64)
    lib().oq_split_attention(fmt.bits, d, int(fmt.hybrid), _p(q), B, Hq, Hkv, _p(kp), _p(vp),
                             kp.shape[1], n_packed, _p(kres), _p(vres), res_cap, n_res, sm, S,
                             _p(po), _p(pl), n_threads or default_threads())
    return po, pl


def combine(part_o: np.ndarray, part_lse: np.ndarray) -> np.ndarray:
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    B, Hq, S, d = po.shape
    out = np.zeros((B, Hq, d), np.float64)
    lib().oq_combine(_p(po), _p(pl), B, Hq, d, S, _p(out))
    return out


def split_range(n_packed: int, n_res: int, S: int, s: int) -> tuple[int, int]:
    lo, hi = C.c_int64(), C.c_int64()
    lib().oq_split_range(n_packed, n_res, S, s, C.byref(lo), C.byref(hi))
    return lo.value, hi.value


def key_norm(k16) -> np.ndarray:
    """norm[rows][d] (float32) of key-channel normalization over k16[rows][T][d]."""
    k = as_bits(k16)
    rows, T, d = k.shape
    k = np.ascontiguousarray(k)
    out = np.zeros((rows, d), np.float32)
    lib().oq_key_norm(_p(k), rows, T, T * d, d, d, _p(out))
    return out


def channel_scale(x16, norm, rows_per_norm: int = 1, multiply: bool = False) -> np.ndarray:
    """fp16 bits of x / norm (keys) or x * norm (queries), x16[rows][T][d], per channel,
    norm row r // rows_per_norm."""
    x = np.ascontiguousarray(as_bits(x16))
    rows, T, d = x.shape
    nm = np.ascontiguousarray(norm, np.float32)
    out = np.zeros_like(x)
    lib().oq_channel_scale(_p(x), rows, T, T * d, d, d, _p(nm), rows_per_norm, int(multiply),
                           _p(out), T * d, d)
    return out


# ---- paged cache, ragged lengths, per-token sliding window -------------------------------

def _pool_strides(pool, block_stride, head_stride):
    if block_stride is None or head_stride is None:
        nblk, hkv, bb = pool.shape            # [n_blocks][Hkv][block_bytes]
        return hkv * bb, bb
    return block_stride, head_stride


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def pack_tokens_paged(fmt: Format, src16, B: int, Hkv: int, count, start, pool, table,
                      block_stride=None, head_stride=None):
    """Quantize tokens [0, count[b]) of src16[B*Hkv][T][d] into packed positions
    start[b] + t of each sequence's paged cache; `pool` (uint8) is written in place."""
    src = np.ascontiguousarray(as_bits(src16))
    rows, T, d = src.shape
    assert rows == B * Hkv and pool.dtype == np.uint8 and pool.flags.c_contiguous
    tbl = _i32(table)
    bs, hs = _pool_strides(pool, block_stride, head_stride)
    lib().oq_pack_tokens_paged(fmt.bits, d, int(fmt.hybrid), _p(src), B, Hkv, T * d, d,
                               _p(_i32(count)), _p(_i32(start)), _p(pool), bs, hs, _p(tbl),
                               tbl.shape[1])


def append_evict(fmt: Format, k_new16, v_new16, k_res16, v_res16, n_sink: int, k_pool, v_pool,
                 table, state, block_stride=None, head_stride=None):
    """One decode-step window update with per-token eviction. k_res16/v_res16 (uint16 bits
    or fp16, [B][Hkv][cap][d]), the pools and state ([B][4] int32) are updated in place."""
    B, Hkv, cap, d = k_res16.shape
    for a in (k_res16, v_res16, k_pool, v_pool, state):
        assert a.flags.c_contiguous and a.flags.writeable
    assert state.dtype == np.int32 and state.shape == (B, 4)
    kn = np.ascontiguousarray(as_bits(k_new16))
    vn = np.ascontiguousarray(as_bits(v_new16))
    tbl = _i32(table)
    bs, hs = _pool_strides(k_pool, block_stride, head_stride)
    lib().oq_append_evict(fmt.bits, d, int(fmt.hybrid), _p(kn), _p(vn), _p(k_res16),
                          _p(v_res16), cap, n_sink, _p(k_pool), _p(v_pool), bs, hs, _p(tbl),
                          tbl.shape[1], _p(state), B, Hkv)


def attention_paged(fmt: Format, q16, Hkv: int, k_pool, v_pool, table, state, k_res16, v_res16,
                    sm: float | None = None, S: int = 0, block_stride=None, head_stride=None,
                    n_threads: int | None = None):
    """fp64 attention of every sequence over its own packed tokens (state[b][0] of them,
    through the table) and window slots [0, state[b][1]). S == 0: out[B][Hq][d];
    S >= 1: the split partials (part_o[B][Hq][S][d], part_lse[B][Hq][S])."""
    q = np.ascontiguousarray(as_bits(q16))
    B, Hq, d = q.shape
    kr = np.ascontiguousarray(as_bits(k_res16))
    vr = np.ascontiguousarray(as_bits(v_res16))
    cap = kr.shape[2]
    tbl = _i32(table)
    st = _i32(state)
    bs, hs = _pool_strides(k_pool, block_stride, head_stride)
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    kp = np.ascontiguousarray(k_pool)
    vp = np.ascontiguousarray(v_pool)
    if S == 0:
        out = np.zeros((B, Hq, d), np.float64)
        lse = np.zeros(1, np.float64)
    else:
        out = np.zeros((B, Hq, S, d), np.float64)
        lse = np.zeros((B, Hq, S), np.float64)
    lib().oq_attention_paged(fmt.bits, d, int(fmt.hybrid), _p(q), B, Hq, Hkv, _p(kp), _p(vp),
                             bs, hs, _p(tbl), tbl.shape[1], _p(st), _p(kr), _p(vr), cap, sm, S,
                             _p(out), _p(lse), n_threads or default_threads())
    return out if S == 0 else (out, lse)


def paged_split_range(n_packed: int, n_res: int, S: int, s: int) -> tuple[int, int]:
    lo, hi = C.c_int64(), C.c_int64()
    lib().oq_paged_split_range(n_packed, n_res, S, s, C.byref(lo), C.byref(hi))
    return lo.value, hi.value


# ---- outer-dimension (KIVI-style) grouping -------------------------------------------------

def quantize_pack_outer(fmt: Format, src16, n_threads: int | None = None) -> np.ndarray:
    """Blocks of src16[rows][T][d] (T a multiple of 128) with groups of 32 tokens per
    channel; codes at the inner layout's positions, scale/zero as [4][d] per block."""
    assert not fmt.hybrid, "outer grouping is asymmetric only"
    src = np.ascontiguousarray(as_bits(src16))
    rows, T, d = src.shape
    nb = T // BLOCK
    out = np.zeros((rows, nb * fmt.block_bytes), np.uint8)
    rc = lib().oq_quantize_pack_outer(fmt.bits, d, _p(src), rows, T, T * d, d, _p(out),
                                      out.shape[1], 0)
    if rc != 0:
        raise ValueError("bad arguments")
    return out


def attention_outer(fmt: Format, q16, Hkv: int, kp, vp, n_packed: int, kres16=None,
                    vres16=None, n_res: int = 0, sm: float | None = None,
                    n_threads: int | None = None):
    """attention() over outer-grouped packed blocks."""
    q, B, Hq, d, kp, vp, kres, vres, res_cap = _att_args(fmt, q16, Hkv, kp, vp, n_packed,
                                                         kres16, vres16, n_res)
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    out = np.zeros((B, Hq, d), np.float64)
    lib().oq_attention_outer(fmt.bits, d, _p(q), B, Hq, Hkv, _p(kp), _p(vp), kp.shape[1],
                             n_packed, _p(kres), _p(vres), res_cap, n_res, sm, _p(out),
                             n_threads or default_threads())
    return out


def split_attention_outer(fmt: Format, q16, Hkv: int, kp, vp, n_packed: int, kres16=None,
                          vres16=None, n_res: int = 0, S: int = 1, sm: float | None = None,
                          n_threads: int | None = None):
    q, B, Hq, d, kp, vp, kres, vres, res_cap = _att_args(fmt, q16, Hkv, kp, vp, n_packed,
                                                         kres16, vres16, n_res)
    sm = float(np.float32(1.0 / np.sqrt(d))) if sm is None else sm
    po = np.zeros((B, Hq, S, d), np.float64)
    pl = np.zeros((B, Hq, S), np.float64)
    lib().oq_split_attention_outer(fmt.bits, d, _p(q), B, Hq, Hkv, _p(kp), _p(vp), kp.shape[1],
                                   n_packed, _p(kres), _p(vres), res_cap, n_res, sm, S, _p(po),
                                   _p(pl), n_threads or default_threads())
    return po, pl
