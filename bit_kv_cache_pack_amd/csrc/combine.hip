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

// Four one-wave workgroups per (batch, head), one per quarter of the channels, so that
// 4 * B * Hq workgroups share the (latency-bound) work and no workgroup barrier is needed.
// Lane t owns the channels 4 * (t % 8) .. +3 of its quarter for the splits s = t / 8,
// t / 8 + 8, ...; it takes them eight at a time, issuing the eight lse loads and the eight
// partial-output loads together (one memory round trip per 64 splits: nothing waits for
// the maximum before the outputs are requested), and keeps a running maximum m with
// sum w_s o_s and sum w_s relative to it, rescaled when m grows. The eight lanes that own
// the same four channels then merge their (m, sum w o, sum w) with the same rule over a
// butterfly of lane exchanges (xor 8, 16, 32).
template <bool F16>
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ part_o,
                                                     const float *__restrict__ part_lse, int S,
                                                     void *__restrict__ out)
{
    constexpr int kGroups = 8, kChunk = 8;
    const int64_t bh = blockIdx.x;
    const int quarter = blockIdx.y;
    const int t = threadIdx.x;
    const int cq = t & 7, sg = t >> 3;
    const float *lse = part_lse + bh * S;
    const float4_t *o = reinterpret_cast<const float4_t *>(part_o + bh * (int64_t)S * kHeadDim) +
                        quarter * 8 + cq;
    float m = -INFINITY, ws = 0.0f;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sg; s0 < S; s0 += kGroups * kChunk) {
        float ls[kChunk];
        float4_t x[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int s = s0 + j * kGroups;
            ls[j] = s < S ? lse[s] : -INFINITY;
            x[j] = s < S ? o[(int64_t)s * (kHeadDim / 4)] : float4_t{0.f, 0.f, 0.f, 0.f};
        }
        float mc = m;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) mc = fmaxf(mc, ls[j]);
        if (mc == -INFINITY) continue;
        const float c = m == -INFINITY ? 0.0f : __expf(m - mc);
        acc *= c;
        ws *= c;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const float w = ls[j] == -INFINITY ? 0.0f : __expf(ls[j] - mc);
            acc += w * x[j];
            ws += w;
        }
        m = mc;
    }
    // butterfly over the eight split groups (lanes cq, cq + 8, ..., cq + 56)
#pragma unroll
    for (int d = 8; d < 64; d <<= 1) {
        const float m2 = __shfl_xor(m, d);
        const float w2 = __shfl_xor(ws, d);
        float4_t a2;
#pragma unroll
        for (int k = 0; k < 4; ++k) a2[k] = __shfl_xor(acc[k], d);
        const float M = fmaxf(m, m2);
        const float c1 = m == -INFINITY ? 0.0f : __expf(m - M);
        const float c2 = m2 == -INFINITY ? 0.0f : __expf(m2 - M);
        acc = c1 * acc + c2 * a2;
        ws = c1 * ws + c2 * w2;
        m = M;
    }
    if (t < 8) {
        // a (b, h) whose splits are all empty attended no token: its output is 0
        const float4_t r = ws > 0.0f ? acc / ws : float4_t{0.f, 0.f, 0.f, 0.f};
        const int64_t idx = bh * (kHeadDim / 4) + quarter * 8 + t;
        if (F16) {
            typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
            const half4_t h = {(_Float16)r[0], (_Float16)r[1], (_Float16)r[2], (_Float16)r[3]};
            reinterpret_cast<half4_t *>(out)[idx] = h;
        } else {
            reinterpret_cast<float4_t *>(out)[idx] = r;
        }
    }
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
    const dim3 grid((uint32_t)((int64_t)B * Hq), 4);
    if (out_f16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(64), 0, stream, part_o, part_lse,
                           num_splits, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(64), 0, stream, part_o, part_lse,
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
