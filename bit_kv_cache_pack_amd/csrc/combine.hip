// combine.hip -- merge of split-K partials, and the residual-window append.
//
// The merge is the log-sum-exp combination of split-K flash-decoding (the FP16 decode
// baseline the BitDecoding page, "Tensor Core加速的低比特KV缓存解码系统", compares against
// in sec. 4.2): with M = max_s lse_s and w_s = e^(lse_s - M),
//     out = sum_s w_s o_s / sum_s w_s,
// splits with lse = -inf weighing 0. The append writes a new fp16 token into the recent
// window (InnerQ page, "KV缓存量化技术InnerQ：提升大模型推理效率", sec. 2.3).
#include "kvq_device.h"
#include "kvq_internal.h"

#include <math.h>

namespace kvq {
namespace {

// One workgroup of 128 threads per (batch, head); thread d owns output channel d.
// The lse row is read with uniform (scalar) loads; o rows are 512-byte coalesced reads.
template <bool F16>
__global__ __launch_bounds__(128) void combine_kernel(const float *__restrict__ part_o,
                                                      const float *__restrict__ part_lse, int S,
                                                      void *__restrict__ out)
{
    const int64_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const float *lse = part_lse + bh * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, lse[s]);
    const float *o = part_o + bh * S * kHeadDim + d;
    float acc = 0.0f, wsum = 0.0f;
    int s = 0;
    for (; s + 4 <= S; s += 4) {
        float x[4], w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = o[(int64_t)(s + k) * kHeadDim];
            const float ls = lse[s + k];
            w[k] = ls == -INFINITY ? 0.0f : __expf(ls - M);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc = __builtin_fmaf(w[k], x[k], acc);
            wsum += w[k];
        }
    }
    for (; s < S; ++s) {
        const float ls = lse[s];
        const float w = ls == -INFINITY ? 0.0f : __expf(ls - M);
        acc = __builtin_fmaf(w, o[(int64_t)s * kHeadDim], acc);
        wsum += w;
    }
    const float r = acc / wsum;
    if (F16)
        reinterpret_cast<_Float16 *>(out)[bh * kHeadDim + d] = (_Float16)r;
    else
        reinterpret_cast<float *>(out)[bh * kHeadDim + d] = r;
}

// One workgroup of 32 threads per (batch, kv-head): threads 0..15 copy the K token,
// 16..31 the V token, 16 bytes each.
__global__ __launch_bounds__(32) void append_kernel(const uint16_t *__restrict__ k_new,
                                                    const uint16_t *__restrict__ v_new,
                                                    uint16_t *__restrict__ k_res,
                                                    uint16_t *__restrict__ v_res, int res_cap,
                                                    int slot)
{
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x & 15;
    const bool is_v = threadIdx.x >= 16;
    const uint16_t *src = (is_v ? v_new : k_new) + row * kHeadDim + 8 * t;
    uint16_t *dst = (is_v ? v_res : k_res) + (row * res_cap + slot) * kHeadDim + 8 * t;
    *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
}

}  // namespace

hipError_t launch_combine(const float *part_o, const float *part_lse, int32_t B, int32_t Hq,
                          int32_t num_splits, void *out, int32_t out_f16, hipStream_t stream)
{
    const dim3 grid((uint32_t)((int64_t)B * Hq));
    if (out_f16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(128), 0, stream, part_o, part_lse,
                           num_splits, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(128), 0, stream, part_o, part_lse,
                           num_splits, out);
    return hipGetLastError();
}

hipError_t launch_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                         uint16_t *v_res, int32_t B, int32_t Hkv, int32_t res_cap, int32_t slot,
                         hipStream_t stream)
{
    hipLaunchKernelGGL(append_kernel, dim3((uint32_t)((int64_t)B * Hkv)), dim3(32), 0, stream,
                       k_new, v_new, k_res, v_res, res_cap, slot);
    return hipGetLastError();
}

}  // namespace kvq
