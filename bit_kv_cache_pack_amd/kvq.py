"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Each function has the name and the arguments of the C call. Tensors are passed as device
pointers (torch is used for device memory and streams); `stream=None` means torch's
current stream on the tensors' device. A non-zero status raises KVQError. Every step of
the computation runs in the HIP kernels of libkvq.so; nothing here computes.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB_PATH may name another build of the same ABI (the sanitizer-checked host build)
LIB_PATH = os.environ.get("KVQ_LIB_PATH") or os.path.join(PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN, KVQ_ERR_LAUNCH = \
    0, -1, -2, -3, -4, -5
KVQ_ERR_TOO_LARGE = -6
KVQ_NOALLOC_SCRATCH_BYTES = 8 << 20
KVQ_OUT_F32, KVQ_OUT_F16 = 0, 1
KVQ_SCALE_DIVIDE, KVQ_SCALE_MULTIPLY = 0, 1
_STATUS = {0: "ok", -1: "null pointer", -2: "bad shape or stride",
           -3: "unsupported format or shape", -4: "misaligned pointer or stride",
           -5: "kernel launch failed",
           -6: "sizes exceed the fixed scratch of the allocation-free call"}

EXPORTED = ("kvq_quantize_pack", "kvq_decode_attention", "kvq_decode_attention_knorm",
            "kvq_decode_attention_valu", "kvq_decode_attention_fp16", "kvq_combine",
            "kvq_append_residual", "kvq_key_norm", "kvq_channel_scale", "kvq_pack_tokens_paged",
            "kvq_append_evict", "kvq_decode_attention_paged", "kvq_quantize_pack_outer",
            "kvq_decode_attention_outer", "kvq_decode_attention_append",
            "kvq_decode_attention_fused", "kvq_decode_attention_paged_fused",
            "kvq_decode_attention_fused_noalloc", "kvq_stream_read",
            "kvq_decode_attention_paged_append")
# exported calls that return a size rather than a status
EXPORTED_SIZE = ("kvq_decode_workspace_bytes",)


class KVQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_STATUS.get(status, 'unknown status')} ({status})")
        self.status = status


class kvq_format(C.Structure):
    _fields_ = [("bits", C.c_int32), ("head_dim", C.c_int32), ("group", C.c_int32),
                ("hybrid", C.c_int32), ("block_tokens", C.c_int32)]


_FMT_CACHE: dict = {}


@dataclass(frozen=True)
class Format:
    """Python view of kvq_format with the header's size helpers."""
    bits: int
    head_dim: int = 128
    hybrid: bool = False
    group: int = 32
    block_tokens: int = 128

    def c(self) -> kvq_format:
        f = _FMT_CACHE.get(self)
        if f is None:
            f = _FMT_CACHE[self] = kvq_format(self.bits, self.head_dim, self.group,
                                              int(self.hybrid), self.block_tokens)
        return f

    @staticmethod
    def _a64(v: int) -> int:
        return (v + 63) // 64 * 64

    @property
    def codes_bytes(self) -> int:
        return self.block_tokens * self.head_dim * self.bits // 8

    @property
    def sz_offset(self) -> int:
        return self._a64(self.codes_bytes)

    @property
    def sz_bytes(self) -> int:
        return self.block_tokens * (self.head_dim // self.group) * 4

    @property
    def flag_offset(self) -> int:
        return self._a64(self.sz_offset + self.sz_bytes)

    @property
    def flag_bytes(self) -> int:
        return (self.block_tokens * (self.head_dim // self.group) + 7) // 8 if self.hybrid else 0

    @property
    def block_bytes(self) -> int:
        return self._a64(self.flag_offset + self.flag_bytes)


_lib = None


def lib():
    """Load libkvq.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_kv_cache_pack_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        fp = C.POINTER(kvq_format)
        L.kvq_quantize_pack.argtypes = [fp, vp, i64, i32, i64, i64, vp, i64, i32, vp]
        L.kvq_decode_attention.argtypes = [fp, vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, i32,
                                           i32, f32, i32, vp, vp, vp]
        L.kvq_decode_attention_valu.argtypes = L.kvq_decode_attention.argtypes
        L.kvq_decode_attention_outer.argtypes = L.kvq_decode_attention.argtypes
        L.kvq_quantize_pack_outer.argtypes = L.kvq_quantize_pack.argtypes
        L.kvq_decode_attention_knorm.argtypes = [fp, vp, vp, i32, i32, i32, vp, vp, i64, i32,
                                                 vp, vp, i32, i32, f32, i32, vp, vp, vp]
        L.kvq_decode_attention_fp16.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, f32, i32, vp,
                                                vp, vp]
        L.kvq_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp]
        L.kvq_decode_attention_append.argtypes = [fp, vp, i32, i32, i32, vp, vp, i64, i32, vp,
                                                  vp, i32, i32, vp, vp, f32, i32, vp, vp, vp]
        L.kvq_append_residual.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.kvq_stream_read.argtypes = [C.POINTER(vp), C.POINTER(i64), i32, vp, vp]
        L.kvq_key_norm.argtypes = [vp, i64, i32, i64, i64, i32, vp, vp]
        L.kvq_channel_scale.argtypes = [vp, i64, i32, i64, i64, i32, vp, i64, i32, vp, i64, i64,
                                        vp]
        L.kvq_pack_tokens_paged.argtypes = [fp, vp, i32, i32, i64, i64, vp, vp, i32, vp, i64,
                                            i64, i64, vp, i32, vp]
        L.kvq_append_evict.argtypes = [fp, vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, i64, vp,
                                       i32, vp, i32, i32, vp]
        L.kvq_decode_attention_paged.argtypes = [fp, vp, i32, i32, i32, vp, vp, i64, i64, i64,
                                                 vp, i32, vp, vp, vp, i32, vp, f32, i32, vp, vp,
                                                 vp]
        L.kvq_decode_attention_paged_append.argtypes = [fp, vp, i32, i32, i32, vp, vp, i64, i64,
                                                        i64, vp, i32, vp, vp, vp, vp, i32, i32,
                                                        vp, vp, vp, f32, i32, vp, vp, vp]
        L.kvq_decode_attention_fused.argtypes = [fp, vp, vp, i32, i32, i32, vp, vp, i64, i32,
                                                 vp, vp, i32, i32, vp, vp, f32, i32, vp, i64,
                                                 vp, i32, vp]
        L.kvq_decode_attention_paged_fused.argtypes = [fp, vp, i32, i32, i32, vp, vp, i64, i64,
                                                       i64, vp, i32, vp, vp, vp, i32, vp, f32,
                                                       i32, vp, i64, vp, i32, vp]
        L.kvq_decode_attention_fused_noalloc.argtypes = [fp, vp, vp, i32, i32, i32, vp, vp, i64,
                                                         i32, vp, vp, i32, i32, vp, vp, f32, i32,
                                                         vp, i32, vp]
        L.kvq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.kvq_decode_workspace_bytes.restype = i64
        for n in EXPORTED:
            getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    dev = next((t.device for t in tensors if hasattr(t, "device") and t.device.type == "cuda"),
               None)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(fn: str, st: int):
    if st != KVQ_OK:
        raise KVQError(fn, st)


def kvq_quantize_pack(fmt: Format, src_fp16, n_rows: int, n_tokens: int, src_row_stride: int,
                      src_tok_stride: int, dst_packed, dst_row_stride_bytes: int,
                      dst_first_block: int, stream=None):
    f = fmt.c()
    st = lib().kvq_quantize_pack(C.byref(f), _ptr(src_fp16), n_rows, n_tokens, src_row_stride,
                                 src_tok_stride, _ptr(dst_packed), dst_row_stride_bytes,
                                 dst_first_block, _stream(stream, src_fp16, dst_packed))
    _check("kvq_quantize_pack", st)


def kvq_decode_attention(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed, v_packed,
                         packed_row_stride_bytes: int, n_packed_tokens: int, k_res_fp16,
                         v_res_fp16, res_capacity: int, n_res: int, sm_scale: float,
                         num_splits: int, part_o, part_lse, stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention(C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_packed),
                                    _ptr(v_packed), packed_row_stride_bytes, n_packed_tokens,
                                    _ptr(k_res_fp16), _ptr(v_res_fp16), res_capacity, n_res,
                                    float(sm_scale), num_splits, _ptr(part_o), _ptr(part_lse),
                                    _stream(stream, q_fp16))
    _check("kvq_decode_attention", st)


def kvq_decode_attention_append(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed,
                                v_packed, packed_row_stride_bytes: int, n_packed_tokens: int,
                                k_res_fp16, v_res_fp16, res_capacity: int, n_res: int, k_new_fp16,
                                v_new_fp16, sm_scale: float, num_splits: int, part_o, part_lse,
                                stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_append(C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_packed),
                                           _ptr(v_packed), packed_row_stride_bytes,
                                           n_packed_tokens, _ptr(k_res_fp16), _ptr(v_res_fp16),
                                           res_capacity, n_res, _ptr(k_new_fp16),
                                           _ptr(v_new_fp16), float(sm_scale), num_splits,
                                           _ptr(part_o), _ptr(part_lse), _stream(stream, q_fp16))
    _check("kvq_decode_attention_append", st)


def kvq_quantize_pack_outer(fmt: Format, src_fp16, n_rows: int, n_tokens: int,
                            src_row_stride: int, src_tok_stride: int, dst_packed,
                            dst_row_stride_bytes: int, dst_first_block: int, stream=None):
    f = fmt.c()
    st = lib().kvq_quantize_pack_outer(C.byref(f), _ptr(src_fp16), n_rows, n_tokens,
                                       src_row_stride, src_tok_stride, _ptr(dst_packed),
                                       dst_row_stride_bytes, dst_first_block,
                                       _stream(stream, src_fp16, dst_packed))
    _check("kvq_quantize_pack_outer", st)


def kvq_decode_attention_outer(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed,
                               v_packed, packed_row_stride_bytes: int, n_packed_tokens: int,
                               k_res_fp16, v_res_fp16, res_capacity: int, n_res: int,
                               sm_scale: float, num_splits: int, part_o, part_lse, stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_outer(C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_packed),
                                          _ptr(v_packed), packed_row_stride_bytes,
                                          n_packed_tokens, _ptr(k_res_fp16), _ptr(v_res_fp16),
                                          res_capacity, n_res, float(sm_scale), num_splits,
                                          _ptr(part_o), _ptr(part_lse), _stream(stream, q_fp16))
    _check("kvq_decode_attention_outer", st)


def kvq_decode_attention_knorm(fmt: Format, q_fp16, key_norm, B: int, Hq: int, Hkv: int,
                               k_packed, v_packed, packed_row_stride_bytes: int,
                               n_packed_tokens: int, k_res_fp16, v_res_fp16, res_capacity: int,
                               n_res: int, sm_scale: float, num_splits: int, part_o, part_lse,
                               stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_knorm(C.byref(f), _ptr(q_fp16), _ptr(key_norm), B, Hq, Hkv,
                                          _ptr(k_packed), _ptr(v_packed),
                                          packed_row_stride_bytes, n_packed_tokens,
                                          _ptr(k_res_fp16), _ptr(v_res_fp16), res_capacity,
                                          n_res, float(sm_scale), num_splits, _ptr(part_o),
                                          _ptr(part_lse), _stream(stream, q_fp16))
    _check("kvq_decode_attention_knorm", st)


def kvq_decode_attention_valu(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed,
                              v_packed, packed_row_stride_bytes: int, n_packed_tokens: int,
                              k_res_fp16, v_res_fp16, res_capacity: int, n_res: int,
                              sm_scale: float, num_splits: int, part_o, part_lse, stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_valu(C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_packed),
                                         _ptr(v_packed), packed_row_stride_bytes,
                                         n_packed_tokens, _ptr(k_res_fp16), _ptr(v_res_fp16),
                                         res_capacity, n_res, float(sm_scale), num_splits,
                                         _ptr(part_o), _ptr(part_lse), _stream(stream, q_fp16))
    _check("kvq_decode_attention_valu", st)


def kvq_decode_attention_fp16(q_fp16, B: int, Hq: int, Hkv: int, k_fp16, v_fp16,
                              row_stride_tokens: int, n_tokens: int, sm_scale: float,
                              num_splits: int, part_o, part_lse, stream=None):
    st = lib().kvq_decode_attention_fp16(_ptr(q_fp16), B, Hq, Hkv, _ptr(k_fp16), _ptr(v_fp16),
                                         row_stride_tokens, n_tokens, float(sm_scale),
                                         num_splits, _ptr(part_o), _ptr(part_lse),
                                         _stream(stream, q_fp16))
    _check("kvq_decode_attention_fp16", st)


def kvq_combine(part_o, part_lse, B: int, Hq: int, head_dim: int, num_splits: int, out,
                out_dtype: int = KVQ_OUT_F32, stream=None):
    st = lib().kvq_combine(_ptr(part_o), _ptr(part_lse), B, Hq, head_dim, num_splits, _ptr(out),
                           out_dtype, _stream(stream, part_o))
    _check("kvq_combine", st)


def kvq_append_residual(k_new, v_new, k_res, v_res, B: int, Hkv: int, head_dim: int,
                        res_capacity: int, slot: int, stream=None):
    st = lib().kvq_append_residual(_ptr(k_new), _ptr(v_new), _ptr(k_res), _ptr(v_res), B, Hkv,
                                   head_dim, res_capacity, slot, _stream(stream, k_new))
    _check("kvq_append_residual", st)


def kvq_stream_read(bufs, sink, stream=None):
    """One streaming read of the device buffers `bufs` (1..4 tensors, read whole)."""
    n = len(bufs)
    ptrs = (C.c_void_p * n)(*[_ptr(b) for b in bufs])
    sizes = (C.c_int64 * n)(*[b.numel() * b.element_size() for b in bufs])
    st = lib().kvq_stream_read(ptrs, sizes, n, _ptr(sink), _stream(stream, sink))
    _check("kvq_stream_read", st)


def kvq_key_norm(k_fp16, n_rows: int, n_tokens: int, row_stride: int, tok_stride: int,
                 head_dim: int, norm, stream=None):
    st = lib().kvq_key_norm(_ptr(k_fp16), n_rows, n_tokens, row_stride, tok_stride, head_dim,
                            _ptr(norm), _stream(stream, norm))
    _check("kvq_key_norm", st)


def kvq_channel_scale(x_fp16, n_rows: int, n_tokens: int, x_row_stride: int,
                      x_tok_stride: int, head_dim: int, norm, rows_per_norm: int, mode: int,
                      y_fp16, y_row_stride: int, y_tok_stride: int, stream=None):
    st = lib().kvq_channel_scale(_ptr(x_fp16), n_rows, n_tokens, x_row_stride, x_tok_stride,
                                 head_dim, _ptr(norm), rows_per_norm, mode, _ptr(y_fp16),
                                 y_row_stride, y_tok_stride, _stream(stream, x_fp16))
    _check("kvq_channel_scale", st)


def kvq_pack_tokens_paged(fmt: Format, src_fp16, B: int, Hkv: int, src_row_stride: int,
                          src_tok_stride: int, count, start, max_count: int, pool,
                          pool_blocks: int, block_stride_bytes: int, head_stride_bytes: int,
                          block_table, max_blocks: int, stream=None):
    f = fmt.c()
    st = lib().kvq_pack_tokens_paged(C.byref(f), _ptr(src_fp16), B, Hkv, src_row_stride,
                                     src_tok_stride, _ptr(count), _ptr(start), max_count,
                                     _ptr(pool), pool_blocks, block_stride_bytes,
                                     head_stride_bytes, _ptr(block_table), max_blocks,
                                     _stream(stream, src_fp16, pool))
    _check("kvq_pack_tokens_paged", st)


def kvq_append_evict(fmt: Format, k_new, v_new, k_res, v_res, res_capacity: int, n_sink: int,
                     k_pool, v_pool, pool_blocks: int, block_stride_bytes: int,
                     head_stride_bytes: int, block_table, max_blocks: int, state, B: int,
                     Hkv: int, stream=None):
    f = fmt.c()
    st = lib().kvq_append_evict(C.byref(f), _ptr(k_new), _ptr(v_new), _ptr(k_res), _ptr(v_res),
                                res_capacity, n_sink, _ptr(k_pool), _ptr(v_pool), pool_blocks,
                                block_stride_bytes, head_stride_bytes, _ptr(block_table),
                                max_blocks, _ptr(state), B, Hkv, _stream(stream, k_new))
    _check("kvq_append_evict", st)


def kvq_decode_attention_paged(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_pool, v_pool,
                               pool_blocks: int, block_stride_bytes: int,
                               head_stride_bytes: int, block_table, max_blocks: int, state,
                               k_res_fp16, v_res_fp16, res_capacity: int, sm_scale: float,
                               num_splits: int, part_o, part_lse, stream=None, key_norm=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_paged(C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_pool),
                                          _ptr(v_pool), pool_blocks, block_stride_bytes,
                                          head_stride_bytes, _ptr(block_table), max_blocks,
                                          _ptr(state), _ptr(k_res_fp16), _ptr(v_res_fp16),
                                          res_capacity, _ptr(key_norm), float(sm_scale),
                                          num_splits, _ptr(part_o), _ptr(part_lse),
                                          _stream(stream, q_fp16))
    _check("kvq_decode_attention_paged", st)


def kvq_decode_attention_paged_append(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_pool,
                                      v_pool, pool_blocks: int, block_stride_bytes: int,
                                      head_stride_bytes: int, block_table, max_blocks: int,
                                      state, state_out, k_res_fp16, v_res_fp16,
                                      res_capacity: int, n_sink: int, k_new, v_new,
                                      sm_scale: float, num_splits: int, part_o, part_lse,
                                      stream=None, key_norm=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_paged_append(
        C.byref(f), _ptr(q_fp16), B, Hq, Hkv, _ptr(k_pool), _ptr(v_pool), pool_blocks,
        block_stride_bytes, head_stride_bytes, _ptr(block_table), max_blocks, _ptr(state),
        _ptr(state_out), _ptr(k_res_fp16), _ptr(v_res_fp16), res_capacity, n_sink, _ptr(k_new),
        _ptr(v_new), _ptr(key_norm), float(sm_scale), num_splits, _ptr(part_o), _ptr(part_lse),
        _stream(stream, q_fp16))
    _check("kvq_decode_attention_paged_append", st)


def kvq_decode_workspace_bytes(B: int, Hq: int, Hkv: int, num_splits: int) -> int:
    n = lib().kvq_decode_workspace_bytes(B, Hq, Hkv, num_splits)
    if n < 0:
        raise KVQError("kvq_decode_workspace_bytes", KVQ_ERR_SHAPE)
    return int(n)


def kvq_decode_attention_fused(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed,
                               v_packed, packed_row_stride_bytes: int, n_packed_tokens: int,
                               k_res_fp16, v_res_fp16, res_capacity: int, n_res: int,
                               sm_scale: float, num_splits: int, workspace, workspace_bytes: int,
                               out, out_dtype: int = KVQ_OUT_F32, key_norm=None, k_new_fp16=None,
                               v_new_fp16=None, stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_fused(C.byref(f), _ptr(q_fp16), _ptr(key_norm), B, Hq, Hkv,
                                          _ptr(k_packed), _ptr(v_packed),
                                          packed_row_stride_bytes, n_packed_tokens,
                                          _ptr(k_res_fp16), _ptr(v_res_fp16), res_capacity,
                                          n_res, _ptr(k_new_fp16), _ptr(v_new_fp16),
                                          float(sm_scale), num_splits, _ptr(workspace),
                                          workspace_bytes, _ptr(out), out_dtype,
                                          _stream(stream, q_fp16))
    _check("kvq_decode_attention_fused", st)


def kvq_decode_attention_fused_noalloc(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_packed,
                                       v_packed, packed_row_stride_bytes: int,
                                       n_packed_tokens: int, k_res_fp16, v_res_fp16,
                                       res_capacity: int, n_res: int, sm_scale: float,
                                       num_splits: int, out, out_dtype: int = KVQ_OUT_F32,
                                       key_norm=None, k_new_fp16=None, v_new_fp16=None,
                                       stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_fused_noalloc(C.byref(f), _ptr(q_fp16), _ptr(key_norm), B,
                                                  Hq, Hkv, _ptr(k_packed), _ptr(v_packed),
                                                  packed_row_stride_bytes, n_packed_tokens,
                                                  _ptr(k_res_fp16), _ptr(v_res_fp16),
                                                  res_capacity, n_res, _ptr(k_new_fp16),
                                                  _ptr(v_new_fp16), float(sm_scale), num_splits,
                                                  _ptr(out), out_dtype, _stream(stream, q_fp16))
    _check("kvq_decode_attention_fused_noalloc", st)


def kvq_decode_attention_paged_fused(fmt: Format, q_fp16, B: int, Hq: int, Hkv: int, k_pool,
                                     v_pool, pool_blocks: int, block_stride_bytes: int,
                                     head_stride_bytes: int, block_table, max_blocks: int, state,
                                     k_res_fp16, v_res_fp16, res_capacity: int, sm_scale: float,
                                     num_splits: int, workspace, workspace_bytes: int, out,
                                     out_dtype: int = KVQ_OUT_F32, key_norm=None, stream=None):
    f = fmt.c()
    st = lib().kvq_decode_attention_paged_fused(C.byref(f), _ptr(q_fp16), B, Hq, Hkv,
                                                _ptr(k_pool), _ptr(v_pool), pool_blocks,
                                                block_stride_bytes, head_stride_bytes,
                                                _ptr(block_table), max_blocks, _ptr(state),
                                                _ptr(k_res_fp16), _ptr(v_res_fp16), res_capacity,
                                                _ptr(key_norm), float(sm_scale), num_splits,
                                                _ptr(workspace), workspace_bytes, _ptr(out),
                                                out_dtype, _stream(stream, q_fp16))
    _check("kvq_decode_attention_paged_fused", st)


def suggest_splits(B: int, Hkv: int, n_tokens: int, cu_count: int = 256) -> int:
    """Same rule as the header's kvq_suggest_splits."""
    rows = B * Hkv
    tiles = n_tokens // 32
    cap = tiles // 8
    if rows >= 1 and 2 * rows <= cu_count and tiles <= 128 * (cu_count // rows):
        want = cu_count // rows
    else:
        want = (3 * cu_count + rows - 1) // rows
        if tiles < 64 * want:
            want = (2 * cu_count + rows - 1) // rows
        elif want >= 2:
            want += 1
    return int(max(1, min(256, min(want, cap))))


def suggest_splits_paged(total_packed: int, max_packed: int, Hkv: int, cu_count: int = 256) -> int:
    """Same rule as the header's kvq_suggest_splits_paged."""
    if total_packed < 1 or max_packed < 1:
        return 1
    s = (4 * cu_count * max_packed + total_packed * Hkv - 1) // (total_packed * Hkv)
    s = min(s, max_packed // 32 // 8)
    return int(max(1, min(256, s)))
