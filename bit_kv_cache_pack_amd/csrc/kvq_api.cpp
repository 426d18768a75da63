// kvq_api.cpp -- the extern "C" boundary of libkvq: argument validation, then launches.
// Every check runs on the host before anything is enqueued; see include/kvq.h for the
// contract of each call.
#include "kvq.h"

#include <math.h>

#include "kvq_internal.h"

namespace {

bool aligned64(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 63u) == 0; }

kvq_status check_format(const kvq_format *f)
{
    if (!f) return KVQ_ERR_NULL;
    if (f->bits < 2 || f->bits > 4 || f->group != 32 || f->block_tokens != 128 ||
        (f->hybrid != 0 && f->hybrid != 1))
        return KVQ_ERR_UNSUPPORTED;
    if (f->head_dim <= 0 || f->head_dim % 32 != 0) return KVQ_ERR_SHAPE;
    if (f->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

kvq_status launched(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

}  // namespace

namespace {

kvq_status quantize_common(const kvq_format *fmt, const void *src_fp16, int64_t n_rows,
                           int32_t n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                           void *dst_packed, int64_t dst_row_stride_bytes,
                           int32_t dst_first_block, hipStream_t stream, bool outer)
{
    kvq_status st = check_format(fmt);
    if (st != KVQ_OK) return st;
    if (outer && fmt->hybrid) return KVQ_ERR_UNSUPPORTED;
    if (!src_fp16 || !dst_packed) return KVQ_ERR_NULL;
    if (n_rows < 1 || n_tokens < 128 || n_tokens % 128 != 0 || dst_first_block < 0)
        return KVQ_ERR_SHAPE;
    if (src_tok_stride < fmt->head_dim || src_row_stride < 0) return KVQ_ERR_SHAPE;
    if (src_row_stride % 8 != 0 || src_tok_stride % 8 != 0) return KVQ_ERR_ALIGN;
    if (!aligned64(src_fp16) || !aligned64(dst_packed) || dst_row_stride_bytes % 64 != 0)
        return KVQ_ERR_ALIGN;
    const int64_t bb = kvq_block_bytes(fmt);
    const int64_t nb = n_tokens / 128;
    if (dst_row_stride_bytes < ((int64_t)dst_first_block + nb) * bb) return KVQ_ERR_SHAPE;
    if (n_rows * nb > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (outer) {
        return launched(kvq::launch_quantize_pack_outer(
            fmt->bits, static_cast<const uint16_t *>(src_fp16), n_rows, n_tokens, src_row_stride,
            src_tok_stride, static_cast<uint8_t *>(dst_packed), dst_row_stride_bytes,
            dst_first_block, (int32_t)bb, (int32_t)kvq_sz_offset(fmt), stream));
    }
    return launched(kvq::launch_quantize_pack(
        fmt->bits, fmt->hybrid, static_cast<const uint16_t *>(src_fp16), n_rows, n_tokens,
        src_row_stride, src_tok_stride, static_cast<uint8_t *>(dst_packed), dst_row_stride_bytes,
        dst_first_block, (int32_t)bb, (int32_t)kvq_sz_offset(fmt), (int32_t)kvq_flag_offset(fmt),
        stream));
}

}  // namespace

extern "C" {

kvq_status kvq_quantize_pack(const kvq_format *fmt, const void *src_fp16, int64_t n_rows,
                             int32_t n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                             void *dst_packed, int64_t dst_row_stride_bytes,
                             int32_t dst_first_block, hipStream_t stream)
{
    return quantize_common(fmt, src_fp16, n_rows, n_tokens, src_row_stride, src_tok_stride,
                           dst_packed, dst_row_stride_bytes, dst_first_block, stream, false);
}

kvq_status kvq_quantize_pack_outer(const kvq_format *fmt, const void *src_fp16, int64_t n_rows,
                                   int32_t n_tokens, int64_t src_row_stride,
                                   int64_t src_tok_stride, void *dst_packed,
                                   int64_t dst_row_stride_bytes, int32_t dst_first_block,
                                   hipStream_t stream)
{
    return quantize_common(fmt, src_fp16, n_rows, n_tokens, src_row_stride, src_tok_stride,
                           dst_packed, dst_row_stride_bytes, dst_first_block, stream, true);
}

}  // extern "C"

namespace {

// Where a decode call leaves its result: the split partials (part_o, part_lse), or, for the
// fused calls, the merged output (out, out_dtype) with the workspace of the in-launch merge.
struct DecodeSink {
    float *part_o = nullptr, *part_lse = nullptr;
    void *out = nullptr;
    int32_t out_dtype = 0;
    void *ws = nullptr;
    int64_t ws_bytes = 0;
    bool fused = false;
    bool noalloc = false;     // records in the library's scratch array (ws unused)
};

DecodeSink partials(float *part_o, float *part_lse)
{
    DecodeSink k;
    k.part_o = part_o;
    k.part_lse = part_lse;
    return k;
}

DecodeSink merged(void *out, int32_t out_dtype, void *ws, int64_t ws_bytes)
{
    DecodeSink k;
    k.out = out;
    k.out_dtype = out_dtype;
    k.ws = ws;
    k.ws_bytes = ws_bytes;
    k.fused = true;
    return k;
}

// checks of the result arguments shared by every decode call
kvq_status check_sink(const DecodeSink &k, int32_t B, int32_t Hq, int32_t Hkv, int32_t S)
{
    if (!k.fused) {
        if (!k.part_o || !k.part_lse) return KVQ_ERR_NULL;
        if (!aligned64(k.part_o) || !aligned64(k.part_lse)) return KVQ_ERR_ALIGN;
        return KVQ_OK;
    }
    if (!k.out) return KVQ_ERR_NULL;
    if (k.out_dtype != KVQ_OUT_F32 && k.out_dtype != KVQ_OUT_F16) return KVQ_ERR_UNSUPPORTED;
    if (!aligned64(k.out)) return KVQ_ERR_ALIGN;
    const int64_t need = kvq::fused_workspace_bytes(B, Hq, Hkv, S);
    if (k.noalloc) return need > KVQ_NOALLOC_SCRATCH_BYTES ? KVQ_ERR_TOO_LARGE : KVQ_OK;
    if (need > 0) {
        if (!k.ws) return KVQ_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(k.ws) & 255u) != 0) return KVQ_ERR_ALIGN;
        if (k.ws_bytes < need) return KVQ_ERR_SHAPE;
    }
    return KVQ_OK;
}

void fill_sink(kvq::DecodeParams &p, const DecodeSink &k)
{
    p.part_o = k.part_o;
    p.part_lse = k.part_lse;
    p.out = k.out;
    p.out_f16 = k.out_dtype == KVQ_OUT_F16;
    p.ws = k.ws;
}

kvq_status decode_common(const kvq_format *fmt, const void *q_fp16, int32_t B, int32_t Hq,
                         int32_t Hkv, const void *k_packed, const void *v_packed,
                         int64_t packed_row_stride_bytes, int32_t n_packed_tokens,
                         const void *k_res_fp16, const void *v_res_fp16, int32_t res_capacity,
                         int32_t n_res, float sm_scale, int32_t num_splits,
                         const DecodeSink &sink, hipStream_t stream, int kind,
                         const float *qnorm = nullptr, const void *k_new = nullptr,
                         const void *v_new = nullptr)
{
    // kind: 0 the MFMA kernel, 1 the VALU comparison kernel, 2 outer-grouped blocks
    if (kind == 2 && fmt && fmt->hybrid) return KVQ_ERR_UNSUPPORTED;
    kvq_status st = check_format(fmt);
    if (st != KVQ_OK) return st;
    if (!q_fp16) return KVQ_ERR_NULL;
    if (n_packed_tokens > 0 && (!k_packed || !v_packed)) return KVQ_ERR_NULL;
    if (n_res > 0 && (!k_res_fp16 || !v_res_fp16)) return KVQ_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return KVQ_ERR_SHAPE;
    if (n_packed_tokens < 0 || n_packed_tokens % 128 != 0) return KVQ_ERR_SHAPE;
    if (n_res < 0 || res_capacity < 0 || n_res > res_capacity) return KVQ_ERR_SHAPE;
    if ((int64_t)n_packed_tokens + n_res <= 0) return KVQ_ERR_SHAPE;
    if (num_splits < 1 || num_splits > 1024) return KVQ_ERR_SHAPE;
    if (!isfinite(sm_scale)) return KVQ_ERR_SHAPE;
    if ((int64_t)B * Hkv > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if ((int64_t)B * Hq * fmt->head_dim * 2 > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
    if (Hq / Hkv > 16) return KVQ_ERR_UNSUPPORTED;
    st = check_sink(sink, B, Hq, Hkv, num_splits);
    if (st != KVQ_OK) return st;
    const int64_t bb = kvq_block_bytes(fmt);
    if (n_packed_tokens > 0) {
        if (packed_row_stride_bytes % 64 != 0) return KVQ_ERR_ALIGN;
        if (packed_row_stride_bytes < (int64_t)(n_packed_tokens / 128) * bb) return KVQ_ERR_SHAPE;
        if ((int64_t)(n_packed_tokens / 128) * bb > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
        if (!aligned64(k_packed) || !aligned64(v_packed)) return KVQ_ERR_ALIGN;
    }
    if (n_res > 0 && (!aligned64(k_res_fp16) || !aligned64(v_res_fp16))) return KVQ_ERR_ALIGN;
    if (!aligned64(q_fp16)) return KVQ_ERR_ALIGN;
    kvq::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q_fp16);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.kp = static_cast<const uint8_t *>(k_packed);
    p.vp = static_cast<const uint8_t *>(v_packed);
    p.row_stride = packed_row_stride_bytes;
    p.n_packed = n_packed_tokens;
    p.kres = static_cast<const uint16_t *>(k_res_fp16);
    p.vres = static_cast<const uint16_t *>(v_res_fp16);
    p.res_cap = res_capacity;
    p.n_res = n_res;
    p.sm_scale = sm_scale;
    p.num_splits = num_splits;
    fill_sink(p, sink);
    p.bits = fmt->bits;
    p.block_bytes = (int32_t)bb;
    p.sz_off = (int32_t)kvq_sz_offset(fmt);
    p.qnorm = qnorm;
    p.knew = static_cast<const uint16_t *>(k_new);
    p.vnew = static_cast<const uint16_t *>(v_new);
    if (sink.noalloc) return launched(kvq::launch_decode_fused_noalloc(p, stream));
    if (sink.fused) return launched(kvq::launch_decode_fused(p, stream));
    if (kind == 2) return launched(kvq::launch_decode_outer(p, stream));
    return launched(kind == 1 ? kvq::launch_decode_valu(p, stream) : kvq::launch_decode(p, stream));
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                int32_t Hq, int32_t Hkv, const void *k_packed,
                                const void *v_packed, int64_t packed_row_stride_bytes,
                                int32_t n_packed_tokens, const void *k_res_fp16,
                                const void *v_res_fp16, int32_t res_capacity, int32_t n_res,
                                float sm_scale, int32_t num_splits, float *part_o,
                                float *part_lse, hipStream_t stream)
{
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, partials(part_o, part_lse), stream, 0);
}

kvq_status kvq_decode_attention_append(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                       int32_t Hq, int32_t Hkv, const void *k_packed,
                                       const void *v_packed, int64_t packed_row_stride_bytes,
                                       int32_t n_packed_tokens, void *k_res_fp16,
                                       void *v_res_fp16, int32_t res_capacity, int32_t n_res,
                                       const void *k_new_fp16, const void *v_new_fp16,
                                       float sm_scale, int32_t num_splits, float *part_o,
                                       float *part_lse, hipStream_t stream)
{
    if (!k_new_fp16 || !v_new_fp16 || !k_res_fp16 || !v_res_fp16) return KVQ_ERR_NULL;
    if (n_res < 1) return KVQ_ERR_SHAPE;
    if (!aligned64(k_new_fp16) || !aligned64(v_new_fp16)) return KVQ_ERR_ALIGN;
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, partials(part_o, part_lse), stream, 0, nullptr, k_new_fp16,
                         v_new_fp16);
}

kvq_status kvq_decode_attention_knorm(const kvq_format *fmt, const void *q_fp16,
                                      const float *key_norm, int32_t B, int32_t Hq,
                                      int32_t Hkv, const void *k_packed, const void *v_packed,
                                      int64_t packed_row_stride_bytes, int32_t n_packed_tokens,
                                      const void *k_res_fp16, const void *v_res_fp16,
                                      int32_t res_capacity, int32_t n_res, float sm_scale,
                                      int32_t num_splits, float *part_o, float *part_lse,
                                      hipStream_t stream)
{
    if (!key_norm) return KVQ_ERR_NULL;
    if (!aligned64(key_norm)) return KVQ_ERR_ALIGN;
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, partials(part_o, part_lse), stream, 0, key_norm);
}

kvq_status kvq_decode_attention_fused(const kvq_format *fmt, const void *q_fp16,
                                      const float *key_norm, int32_t B, int32_t Hq, int32_t Hkv,
                                      const void *k_packed, const void *v_packed,
                                      int64_t packed_row_stride_bytes, int32_t n_packed_tokens,
                                      void *k_res_fp16, void *v_res_fp16, int32_t res_capacity,
                                      int32_t n_res, const void *k_new_fp16,
                                      const void *v_new_fp16, float sm_scale, int32_t num_splits,
                                      void *workspace, int64_t workspace_bytes, void *out,
                                      int32_t out_dtype, hipStream_t stream)
{
    if ((k_new_fp16 == nullptr) != (v_new_fp16 == nullptr)) return KVQ_ERR_NULL;
    if (k_new_fp16) {
        if (!k_res_fp16 || !v_res_fp16) return KVQ_ERR_NULL;
        if (n_res < 1) return KVQ_ERR_SHAPE;
        if (!aligned64(k_new_fp16) || !aligned64(v_new_fp16)) return KVQ_ERR_ALIGN;
    }
    if (key_norm && !aligned64(key_norm)) return KVQ_ERR_ALIGN;
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, merged(out, out_dtype, workspace, workspace_bytes), stream,
                         0, key_norm, k_new_fp16, v_new_fp16);
}

kvq_status kvq_decode_attention_fused_noalloc(const kvq_format *fmt, const void *q_fp16,
                                              const float *key_norm, int32_t B, int32_t Hq,
                                              int32_t Hkv, const void *k_packed,
                                              const void *v_packed,
                                              int64_t packed_row_stride_bytes,
                                              int32_t n_packed_tokens, void *k_res_fp16,
                                              void *v_res_fp16, int32_t res_capacity,
                                              int32_t n_res, const void *k_new_fp16,
                                              const void *v_new_fp16, float sm_scale,
                                              int32_t num_splits, void *out, int32_t out_dtype,
                                              hipStream_t stream)
{
    if ((k_new_fp16 == nullptr) != (v_new_fp16 == nullptr)) return KVQ_ERR_NULL;
    if (k_new_fp16) {
        if (!k_res_fp16 || !v_res_fp16) return KVQ_ERR_NULL;
        if (n_res < 1) return KVQ_ERR_SHAPE;
        if (!aligned64(k_new_fp16) || !aligned64(v_new_fp16)) return KVQ_ERR_ALIGN;
    }
    if (key_norm && !aligned64(key_norm)) return KVQ_ERR_ALIGN;
    DecodeSink sink = merged(out, out_dtype, nullptr, 0);
    sink.noalloc = true;
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, sink, stream, 0, key_norm, k_new_fp16, v_new_fp16);
}

int64_t kvq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t num_splits)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || num_splits < 1 || num_splits > 1024)
        return -1;
    return kvq::fused_workspace_bytes(B, Hq, Hkv, num_splits);
}

kvq_status kvq_decode_attention_outer(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                      int32_t Hq, int32_t Hkv, const void *k_packed,
                                      const void *v_packed, int64_t packed_row_stride_bytes,
                                      int32_t n_packed_tokens, const void *k_res_fp16,
                                      const void *v_res_fp16, int32_t res_capacity,
                                      int32_t n_res, float sm_scale, int32_t num_splits,
                                      float *part_o, float *part_lse, hipStream_t stream)
{
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, partials(part_o, part_lse), stream, 2);
}

kvq_status kvq_decode_attention_valu(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                     int32_t Hq, int32_t Hkv, const void *k_packed,
                                     const void *v_packed, int64_t packed_row_stride_bytes,
                                     int32_t n_packed_tokens, const void *k_res_fp16,
                                     const void *v_res_fp16, int32_t res_capacity,
                                     int32_t n_res, float sm_scale, int32_t num_splits,
                                     float *part_o, float *part_lse, hipStream_t stream)
{
    return decode_common(fmt, q_fp16, B, Hq, Hkv, k_packed, v_packed, packed_row_stride_bytes,
                         n_packed_tokens, k_res_fp16, v_res_fp16, res_capacity, n_res, sm_scale,
                         num_splits, partials(part_o, part_lse), stream, 1);
}

kvq_status kvq_decode_attention_fp16(const void *q_fp16, int32_t B, int32_t Hq, int32_t Hkv,
                                     const void *k_fp16, const void *v_fp16,
                                     int64_t row_stride_tokens, int32_t n_tokens,
                                     float sm_scale, int32_t num_splits, float *part_o,
                                     float *part_lse, hipStream_t stream)
{
    if (!q_fp16 || !k_fp16 || !v_fp16 || !part_o || !part_lse) return KVQ_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return KVQ_ERR_SHAPE;
    if (n_tokens < 1 || row_stride_tokens < n_tokens) return KVQ_ERR_SHAPE;
    if (num_splits < 1 || num_splits > 1024) return KVQ_ERR_SHAPE;
    if (!isfinite(sm_scale)) return KVQ_ERR_SHAPE;
    if ((int64_t)B * Hkv > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (Hq / Hkv > 16) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * 128 * 2 > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)n_tokens * 128 * 2 > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
    if (row_stride_tokens > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
    if (row_stride_tokens % 2 != 0) return KVQ_ERR_ALIGN;      // 512 B: keeps rows 64-B aligned
    if (!aligned64(q_fp16) || !aligned64(k_fp16) || !aligned64(v_fp16) || !aligned64(part_o) ||
        !aligned64(part_lse))
        return KVQ_ERR_ALIGN;
    kvq::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q_fp16);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.kres = static_cast<const uint16_t *>(k_fp16);
    p.vres = static_cast<const uint16_t *>(v_fp16);
    p.res_cap = (int32_t)row_stride_tokens;
    p.n_res = n_tokens;
    p.sm_scale = sm_scale;
    p.num_splits = num_splits;
    p.part_o = part_o;
    p.part_lse = part_lse;
    return launched(kvq::launch_decode_f16(p, stream));
}

kvq_status kvq_combine(const float *part_o, const float *part_lse, int32_t B, int32_t Hq,
                       int32_t head_dim, int32_t num_splits, void *out, int32_t out_dtype,
                       hipStream_t stream)
{
    if (!part_o || !part_lse || !out) return KVQ_ERR_NULL;
    if (B < 1 || Hq < 1 || num_splits < 1 || num_splits > 1024) return KVQ_ERR_SHAPE;
    if (head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_F16) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (!aligned64(part_o) || !aligned64(part_lse) || !aligned64(out)) return KVQ_ERR_ALIGN;
    return launched(kvq::launch_combine(part_o, part_lse, B, Hq, num_splits, out,
                                        out_dtype == KVQ_OUT_F16, stream));
}

kvq_status kvq_stream_read(const void *const *bufs, const int64_t *bytes, int32_t n, void *sink,
                           hipStream_t stream)
{
    if (!bufs || !bytes || !sink) return KVQ_ERR_NULL;
    if (n < 1 || n > 4) return KVQ_ERR_SHAPE;
    int64_t pieces = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (!bufs[i]) return KVQ_ERR_NULL;
        if (bytes[i] < 16 || bytes[i] % 16 != 0) return KVQ_ERR_SHAPE;
        if (reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0) return KVQ_ERR_ALIGN;
        pieces += (bytes[i] + 65535) / 65536;
    }
    if (pieces > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(sink) % 16 != 0) return KVQ_ERR_ALIGN;
    return launched(kvq::launch_stream_read(bufs, bytes, n, static_cast<uint32_t *>(sink), stream));
}

kvq_status kvq_append_residual(const void *k_new, const void *v_new, void *k_res, void *v_res,
                               int32_t B, int32_t Hkv, int32_t head_dim, int32_t res_capacity,
                               int32_t slot, hipStream_t stream)
{
    if (!k_new || !v_new || !k_res || !v_res) return KVQ_ERR_NULL;
    if (B < 1 || Hkv < 1 || res_capacity < 1 || slot < 0 || slot >= res_capacity)
        return KVQ_ERR_SHAPE;
    if (head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (!aligned64(k_new) || !aligned64(v_new) || !aligned64(k_res) || !aligned64(v_res))
        return KVQ_ERR_ALIGN;
    return launched(kvq::launch_append(
        static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
        static_cast<uint16_t *>(k_res), static_cast<uint16_t *>(v_res), B, Hkv, res_capacity,
        slot, stream));
}

}  // extern "C"

namespace {

// Validate a paged pool's geometry and fill the launcher's description of it.
kvq_status check_pool(const kvq_format *fmt, int32_t Hkv, int64_t pool_blocks,
                      int64_t block_stride, int64_t head_stride, const int32_t *tbl,
                      int32_t max_blocks, kvq::PagedPool &pp)
{
    if (!tbl) return KVQ_ERR_NULL;
    if (pool_blocks < 1 || max_blocks < 1 || block_stride < 1 || head_stride < 1)
        return KVQ_ERR_SHAPE;
    if ((int64_t)max_blocks * 128 > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (block_stride % 64 != 0 || head_stride % 64 != 0) return KVQ_ERR_ALIGN;
    const int64_t bb = kvq_block_bytes(fmt);
    // blocks of one head side by side ([blocks][Hkv][bb]) or heads side by side
    // ([Hkv][blocks][bb]); anything else could overlap
    const bool by_block = head_stride >= bb && block_stride / Hkv >= head_stride;
    const bool by_head = block_stride >= bb && head_stride / pool_blocks >= block_stride;
    if (!by_block && !by_head) return KVQ_ERR_SHAPE;
    pp.bits = fmt->bits;
    pp.hybrid = fmt->hybrid;
    pp.pool_blocks = pool_blocks;
    pp.block_stride = block_stride;
    pp.head_stride = head_stride;
    pp.tbl = tbl;
    pp.max_blocks = max_blocks;
    pp.block_bytes = (int32_t)bb;
    pp.sz_off = (int32_t)kvq_sz_offset(fmt);
    pp.flag_off = (int32_t)kvq_flag_offset(fmt);
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_pack_tokens_paged(const kvq_format *fmt, const void *src_fp16, int32_t B,
                                 int32_t Hkv, int64_t src_row_stride, int64_t src_tok_stride,
                                 const int32_t *count, const int32_t *start, int32_t max_count,
                                 void *pool, int64_t pool_blocks, int64_t block_stride_bytes,
                                 int64_t head_stride_bytes, const int32_t *block_table,
                                 int32_t max_blocks, hipStream_t stream)
{
    kvq_status st = check_format(fmt);
    if (st != KVQ_OK) return st;
    if (!src_fp16 || !count || !start || !pool) return KVQ_ERR_NULL;
    if (B < 1 || Hkv < 1 || max_count < 0) return KVQ_ERR_SHAPE;
    if (src_row_stride < 0 || src_tok_stride < fmt->head_dim) return KVQ_ERR_SHAPE;
    if (src_row_stride % 8 != 0 || src_tok_stride % 8 != 0) return KVQ_ERR_ALIGN;
    if (!aligned64(src_fp16) || !aligned64(pool)) return KVQ_ERR_ALIGN;
    kvq::PagedPool pp{};
    st = check_pool(fmt, Hkv, pool_blocks, block_stride_bytes, head_stride_bytes, block_table,
                    max_blocks, pp);
    if (st != KVQ_OK) return st;
    if ((int64_t)B * Hkv * ((max_count + 63) / 64) > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    return launched(kvq::launch_pack_tokens_paged(
        pp, static_cast<const uint16_t *>(src_fp16), B, Hkv, src_row_stride, src_tok_stride, count,
        start, max_count, static_cast<uint8_t *>(pool), stream));
}

kvq_status kvq_append_evict(const kvq_format *fmt, const void *k_new, const void *v_new,
                            void *k_res, void *v_res, int32_t res_capacity, int32_t n_sink,
                            void *k_pool, void *v_pool, int64_t pool_blocks,
                            int64_t block_stride_bytes, int64_t head_stride_bytes,
                            const int32_t *block_table, int32_t max_blocks, kvq_seq_state *state,
                            int32_t B, int32_t Hkv, hipStream_t stream)
{
    kvq_status st = check_format(fmt);
    if (st != KVQ_OK) return st;
    if (!k_new || !v_new || !k_res || !v_res || !k_pool || !v_pool || !state) return KVQ_ERR_NULL;
    if (B < 1 || Hkv < 1 || res_capacity < 1 || n_sink < 0 || n_sink >= res_capacity)
        return KVQ_ERR_SHAPE;
    if ((int64_t)B * Hkv > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (!aligned64(k_new) || !aligned64(v_new) || !aligned64(k_res) || !aligned64(v_res) ||
        !aligned64(k_pool) || !aligned64(v_pool) || !aligned64(state))
        return KVQ_ERR_ALIGN;
    kvq::PagedPool pp{};
    st = check_pool(fmt, Hkv, pool_blocks, block_stride_bytes, head_stride_bytes, block_table,
                    max_blocks, pp);
    if (st != KVQ_OK) return st;
    return launched(kvq::launch_append_evict(
        pp, static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
        static_cast<uint16_t *>(k_res), static_cast<uint16_t *>(v_res), res_capacity, n_sink,
        static_cast<uint8_t *>(k_pool), static_cast<uint8_t *>(v_pool),
        reinterpret_cast<int32_t *>(state), B, Hkv, stream));
}

}  // extern "C"

namespace {

// the step's cache update folded into a paged decode (kvq_decode_attention_paged_append)
struct PagedUpdate {
    const void *k_new = nullptr, *v_new = nullptr;
    int32_t n_sink = 0;
    kvq_seq_state *state_out = nullptr;
};

kvq_status paged_common(const kvq_format *fmt, const void *q_fp16, int32_t B, int32_t Hq,
                        int32_t Hkv, const void *k_pool, const void *v_pool, int64_t pool_blocks,
                        int64_t block_stride_bytes, int64_t head_stride_bytes,
                        const int32_t *block_table, int32_t max_blocks,
                        const kvq_seq_state *state, const void *k_res_fp16,
                        const void *v_res_fp16, int32_t res_capacity, const float *key_norm,
                        float sm_scale, int32_t num_splits, const DecodeSink &sink,
                        hipStream_t stream, const PagedUpdate *upd = nullptr)
{
    kvq_status st = check_format(fmt);
    if (st != KVQ_OK) return st;
    if (!q_fp16 || !k_pool || !v_pool || !state || !k_res_fp16 || !v_res_fp16)
        return KVQ_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || res_capacity < 1) return KVQ_ERR_SHAPE;
    if (num_splits < 1 || num_splits > 1024) return KVQ_ERR_SHAPE;
    if (!isfinite(sm_scale)) return KVQ_ERR_SHAPE;
    if ((int64_t)B * Hkv > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (Hq / Hkv > 16) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * fmt->head_dim * 2 > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
    st = check_sink(sink, B, Hq, Hkv, num_splits);
    if (st != KVQ_OK) return st;
    if (!aligned64(q_fp16) || !aligned64(k_pool) || !aligned64(v_pool) || !aligned64(state) ||
        !aligned64(k_res_fp16) || !aligned64(v_res_fp16) || (key_norm && !aligned64(key_norm)))
        return KVQ_ERR_ALIGN;
    kvq::PagedPool pp{};
    st = check_pool(fmt, Hkv, pool_blocks, block_stride_bytes, head_stride_bytes, block_table,
                    max_blocks, pp);
    if (st != KVQ_OK) return st;
    if (upd) {
        if (!upd->k_new || !upd->v_new || !upd->state_out) return KVQ_ERR_NULL;
        if (upd->n_sink < 0 || upd->n_sink >= res_capacity) return KVQ_ERR_SHAPE;
        if (!aligned64(upd->k_new) || !aligned64(upd->v_new) || !aligned64(upd->state_out))
            return KVQ_ERR_ALIGN;
        // the launch reads state while it writes state_out
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(state);
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(upd->state_out);
        const uintptr_t n = (uintptr_t)B * sizeof(kvq_seq_state);
        if (a0 < b0 + n && b0 < a0 + n) return KVQ_ERR_SHAPE;
        if (sink.fused) return KVQ_ERR_UNSUPPORTED;
    }
    kvq::DecodeParams p{};
    p.qnorm = key_norm;
    p.q = static_cast<const uint16_t *>(q_fp16);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.kp = static_cast<const uint8_t *>(k_pool);
    p.vp = static_cast<const uint8_t *>(v_pool);
    p.kres = static_cast<const uint16_t *>(k_res_fp16);
    p.vres = static_cast<const uint16_t *>(v_res_fp16);
    p.res_cap = res_capacity;
    p.sm_scale = sm_scale;
    p.num_splits = num_splits;
    fill_sink(p, sink);
    p.bits = fmt->bits;
    p.block_bytes = pp.block_bytes;
    p.sz_off = pp.sz_off;
    p.tbl = block_table;
    p.max_blocks = max_blocks;
    p.pool_blocks = pool_blocks;
    p.block_stride = block_stride_bytes;
    p.head_stride = head_stride_bytes;
    p.state = reinterpret_cast<const int32_t *>(state);
    if (upd && Hq / Hkv > 4) {
        // more than one head chunk per kv-head row: the update as its own launch on a copy
        // of the state, then the decode (the same result as the folded path)
        int32_t *so = reinterpret_cast<int32_t *>(upd->state_out);
        if (kvq::launch_copy_state(so, reinterpret_cast<const int32_t *>(state), B, stream) !=
            hipSuccess)
            return KVQ_ERR_LAUNCH;
        const hipError_t e = kvq::launch_append_evict(
            pp, static_cast<const uint16_t *>(upd->k_new), static_cast<const uint16_t *>(upd->v_new),
            const_cast<uint16_t *>(p.kres), const_cast<uint16_t *>(p.vres), res_capacity,
            upd->n_sink, const_cast<uint8_t *>(p.kp), const_cast<uint8_t *>(p.vp), so, B, Hkv, stream);
        if (e != hipSuccess) return KVQ_ERR_LAUNCH;
        p.state = so;
        return launched(kvq::launch_decode_paged(p, stream));
    }
    if (upd) {
        p.upd = 1;
        p.knew = static_cast<const uint16_t *>(upd->k_new);
        p.vnew = static_cast<const uint16_t *>(upd->v_new);
        p.n_sink = upd->n_sink;
        p.hybrid = fmt->hybrid;
        p.flag_off = pp.flag_off;
        p.state_out = reinterpret_cast<int32_t *>(upd->state_out);
    }
    return launched(sink.fused ? kvq::launch_decode_paged_fused(p, stream)
                               : kvq::launch_decode_paged(p, stream));
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention_paged(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                      int32_t Hq, int32_t Hkv, const void *k_pool,
                                      const void *v_pool, int64_t pool_blocks,
                                      int64_t block_stride_bytes, int64_t head_stride_bytes,
                                      const int32_t *block_table, int32_t max_blocks,
                                      const kvq_seq_state *state, const void *k_res_fp16,
                                      const void *v_res_fp16, int32_t res_capacity,
                                      const float *key_norm, float sm_scale, int32_t num_splits,
                                      float *part_o, float *part_lse, hipStream_t stream)
{
    return paged_common(fmt, q_fp16, B, Hq, Hkv, k_pool, v_pool, pool_blocks, block_stride_bytes,
                        head_stride_bytes, block_table, max_blocks, state, k_res_fp16, v_res_fp16,
                        res_capacity, key_norm, sm_scale, num_splits, partials(part_o, part_lse),
                        stream);
}

kvq_status kvq_decode_attention_paged_append(
    const kvq_format *fmt, const void *q_fp16, int32_t B, int32_t Hq, int32_t Hkv, void *k_pool,
    void *v_pool, int64_t pool_blocks, int64_t block_stride_bytes, int64_t head_stride_bytes,
    const int32_t *block_table, int32_t max_blocks, const kvq_seq_state *state,
    kvq_seq_state *state_out, void *k_res_fp16, void *v_res_fp16, int32_t res_capacity,
    int32_t n_sink, const void *k_new, const void *v_new, const float *key_norm, float sm_scale,
    int32_t num_splits, float *part_o, float *part_lse, hipStream_t stream)
{
    PagedUpdate u;
    u.k_new = k_new;
    u.v_new = v_new;
    u.n_sink = n_sink;
    u.state_out = state_out;
    return paged_common(fmt, q_fp16, B, Hq, Hkv, k_pool, v_pool, pool_blocks, block_stride_bytes,
                        head_stride_bytes, block_table, max_blocks, state, k_res_fp16, v_res_fp16,
                        res_capacity, key_norm, sm_scale, num_splits, partials(part_o, part_lse),
                        stream, &u);
}

kvq_status kvq_decode_attention_paged_fused(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                            int32_t Hq, int32_t Hkv, const void *k_pool,
                                            const void *v_pool, int64_t pool_blocks,
                                            int64_t block_stride_bytes,
                                            int64_t head_stride_bytes, const int32_t *block_table,
                                            int32_t max_blocks, const kvq_seq_state *state,
                                            const void *k_res_fp16, const void *v_res_fp16,
                                            int32_t res_capacity, const float *key_norm,
                                            float sm_scale, int32_t num_splits, void *workspace,
                                            int64_t workspace_bytes, void *out, int32_t out_dtype,
                                            hipStream_t stream)
{
    return paged_common(fmt, q_fp16, B, Hq, Hkv, k_pool, v_pool, pool_blocks, block_stride_bytes,
                        head_stride_bytes, block_table, max_blocks, state, k_res_fp16, v_res_fp16,
                        res_capacity, key_norm, sm_scale, num_splits,
                        merged(out, out_dtype, workspace, workspace_bytes), stream);
}

kvq_status kvq_key_norm(const void *k_fp16, int64_t n_rows, int32_t n_tokens,
                        int64_t row_stride, int64_t tok_stride, int32_t head_dim, float *norm,
                        hipStream_t stream)
{
    if (!norm || (n_tokens > 0 && !k_fp16)) return KVQ_ERR_NULL;
    if (n_rows < 1 || n_tokens < 0 || row_stride < 0 || tok_stride < head_dim)
        return KVQ_ERR_SHAPE;
    if (head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if ((n_rows * 128 + 255) / 256 > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (n_rows * ((n_tokens + 255) / 256) > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (row_stride % 8 != 0 || tok_stride % 8 != 0) return KVQ_ERR_ALIGN;
    if (!aligned64(norm) || (n_tokens > 0 && !aligned64(k_fp16))) return KVQ_ERR_ALIGN;
    return launched(kvq::launch_key_norm(static_cast<const uint16_t *>(k_fp16), n_rows, n_tokens,
                                         row_stride, tok_stride, norm, stream));
}

kvq_status kvq_channel_scale(const void *x_fp16, int64_t n_rows, int32_t n_tokens,
                             int64_t x_row_stride, int64_t x_tok_stride, int32_t head_dim,
                             const float *norm, int64_t rows_per_norm, int32_t mode,
                             void *y_fp16, int64_t y_row_stride, int64_t y_tok_stride,
                             hipStream_t stream)
{
    if (!x_fp16 || !norm || !y_fp16) return KVQ_ERR_NULL;
    if (n_rows < 1 || n_tokens < 0 || rows_per_norm < 1) return KVQ_ERR_SHAPE;
    if (x_row_stride < 0 || y_row_stride < 0 || x_tok_stride < head_dim ||
        y_tok_stride < head_dim)
        return KVQ_ERR_SHAPE;
    if (head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if (mode != KVQ_SCALE_DIVIDE && mode != KVQ_SCALE_MULTIPLY) return KVQ_ERR_UNSUPPORTED;
    if (n_rows * ((n_tokens + 63) / 64) > 0x7fffffffLL) return KVQ_ERR_SHAPE;
    if (x_row_stride % 8 != 0 || x_tok_stride % 8 != 0 || y_row_stride % 8 != 0 ||
        y_tok_stride % 8 != 0)
        return KVQ_ERR_ALIGN;
    if (!aligned64(x_fp16) || !aligned64(norm) || !aligned64(y_fp16)) return KVQ_ERR_ALIGN;
    return launched(kvq::launch_channel_scale(
        static_cast<const uint16_t *>(x_fp16), n_rows, n_tokens, x_row_stride, x_tok_stride, norm,
        rows_per_norm, mode == KVQ_SCALE_MULTIPLY, static_cast<uint16_t *>(y_fp16), y_row_stride,
        y_tok_stride, stream));
}

}  // extern "C"
