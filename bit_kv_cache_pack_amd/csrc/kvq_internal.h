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
};

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_f16(const DecodeParams &p, hipStream_t stream);

hipError_t launch_combine(const float *part_o, const float *part_lse, int32_t B, int32_t Hq,
                          int32_t num_splits, void *out, int32_t out_f16, hipStream_t stream);

hipError_t launch_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                         uint16_t *v_res, int32_t B, int32_t Hkv, int32_t res_cap, int32_t slot,
                         hipStream_t stream);

hipError_t launch_key_norm(const uint16_t *k, int64_t n_rows, int32_t n_tokens,
                           int64_t row_stride, int64_t tok_stride, float *norm,
                           hipStream_t stream);

hipError_t launch_channel_scale(const uint16_t *x, int64_t n_rows, int32_t n_tokens,
                                int64_t x_row_stride, int64_t x_tok_stride, const float *norm,
                                int64_t rows_per_norm, int multiply, uint16_t *y,
                                int64_t y_row_stride, int64_t y_tok_stride, hipStream_t stream);

}  // namespace kvq
