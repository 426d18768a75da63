// kvq_internal.h -- launchers behind the C ABI (host side). Arguments are validated by
// the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

hipError_t launch_quantize_pack(int bits, int hybrid, const uint16_t *src, int64_t n_rows,
                                int32_t n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                                uint8_t *dst, int64_t dst_row_stride, int32_t first_block,
                                int32_t block_bytes, int32_t sz_off, int32_t flag_off,
                                hipStream_t stream);

struct DecodeParams {
    const uint16_t *q;
    int32_t B, Hq, Hkv;
    const uint8_t *kp, *vp;
    int64_t row_stride;
    int32_t n_packed;
    const uint16_t *kres, *vres;
    int32_t res_cap, n_res;
    float sm_scale;
    int32_t num_splits;
    float *part_o, *part_lse;
    int32_t bits, block_bytes, sz_off;
    const float *qnorm;   // key-channel norms [B*Hkv][128] that q is multiplied by, or null
    // a new token per row [B*Hkv][128] that becomes window slot n_res - 1 (written into the
    // window by the call and attended from here), or null
    const uint16_t *knew, *vnew;
    // paged cache only (kp / vp are the pools; n_packed / n_res come from state per sequence)
    const int32_t *tbl;
    int32_t max_blocks;
    int64_t pool_blocks, block_stride, head_stride;
    const int32_t *state;
    // split merge inside the launch (the fused calls): output and workspace
    void *out;
    int32_t out_f16;
    void *ws;
    // paged only: the step's cache update (kvq_append_evict) folded into the decode: the
    // new token (knew / vnew) enters the window as that call places it, the evicted token
    // (if any) is quantized into the pool, state is only read and the updated state is
    // written to state_out
    int32_t upd, n_sink, hybrid, flag_off;
    int32_t *state_out;
};

// Workspace of the fused split merge: per group (a row's chunk of up to 4 query heads) one
// 2080-byte slot per node below the root of the fan-in-32 split tree (a record, plus the
// counter of the node's parent in the padding of its first child's slot). One level of
// merging up to 32 splits: at llama8b_32k (32 splits) the fused step took 14.45 us against
// 15.41 us with fan-in 8 (two levels), at batch8_2bit_hybrid 43.9 against 44.6 us.
#ifndef KVQ_FANIN
#define KVQ_FANIN 32
#endif
constexpr int32_t kFanIn = KVQ_FANIN;     // children per node of the split tree

inline int32_t fused_records(int32_t S)
{
    int32_t r = 0;
    for (int32_t n = S; n > 1; n = (n + kFanIn - 1) / kFanIn) r += n;
    return r;
}
inline int64_t fused_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S)
{
    const int64_t groups = (int64_t)B * Hkv * ((Hq / Hkv + 3) / 4);
    return groups * (int64_t)fused_records(S) * 2080;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_fused(const DecodeParams &p, hipStream_t stream);
// the fused decode with its records in the library's per-device scratch array (p.ws unused)
hipError_t launch_decode_fused_noalloc(DecodeParams p, hipStream_t stream);
hipError_t launch_decode_paged_fused(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_paged(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_outer(const DecodeParams &p, hipStream_t stream);

hipError_t launch_quantize_pack_outer(int bits, const uint16_t *src, int64_t n_rows,
                                      int32_t n_tokens, int64_t src_row_stride,
                                      int64_t src_tok_stride, uint8_t *dst, int64_t dst_row_stride,
                                      int32_t first_block, int32_t block_bytes, int32_t sz_off,
                                      hipStream_t stream);
hipError_t launch_decode_f16(const DecodeParams &p, hipStream_t stream);

hipError_t launch_combine(const float *part_o, const float *part_lse, int32_t B, int32_t Hq,
                          int32_t num_splits, void *out, int32_t out_f16, hipStream_t stream);

hipError_t launch_stream_read(const void *const *bufs, const int64_t *bytes, int32_t n,
                              uint32_t *sink, hipStream_t stream);

hipError_t launch_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                         uint16_t *v_res, int32_t B, int32_t Hkv, int32_t res_cap, int32_t slot,
                         hipStream_t stream);

// Geometry of a paged packed cache (pool of blocks addressed through a block table).
struct PagedPool {
    int32_t bits, hybrid;
    int64_t pool_blocks, block_stride, head_stride;   // strides in bytes
    const int32_t *tbl;                               // [B][max_blocks]
    int32_t max_blocks;
    int32_t block_bytes, sz_off, flag_off;
};

hipError_t launch_pack_tokens_paged(const PagedPool &pool, const uint16_t *src, int32_t B,
                                    int32_t Hkv, int64_t src_row_stride, int64_t src_tok_stride,
                                    const int32_t *count, const int32_t *start, int32_t max_count,
                                    uint8_t *dst_pool, hipStream_t stream);

// copy of B sequence states (4 int32 each), stream-ordered
hipError_t launch_copy_state(int32_t *dst, const int32_t *src, int32_t B, hipStream_t stream);

hipError_t launch_append_evict(const PagedPool &pool, const uint16_t *k_new,
                               const uint16_t *v_new, uint16_t *k_res, uint16_t *v_res,
                               int32_t res_cap, int32_t n_sink, uint8_t *k_pool, uint8_t *v_pool,
                               int32_t *state, int32_t B, int32_t Hkv, hipStream_t stream);

hipError_t launch_key_norm(const uint16_t *k, int64_t n_rows, int32_t n_tokens,
                           int64_t row_stride, int64_t tok_stride, float *norm,
                           hipStream_t stream);

hipError_t launch_channel_scale(const uint16_t *x, int64_t n_rows, int32_t n_tokens,
                                int64_t x_row_stride, int64_t x_tok_stride, const float *norm,
                                int64_t rows_per_norm, int multiply, uint16_t *y,
                                int64_t y_row_stride, int64_t y_tok_stride, hipStream_t stream);

}  // namespace kvq
