// keynorm.hip -- key-channel normalization (InnerQ page, "KV缓存量化技术InnerQ：提升大模型推理
// 效率", sec. 2.4): over the prefill keys of one (batch, kv-head) row, channel c gets
// norm_c = sqrt(max_t |K[t][c]|); keys are divided by it before they are quantized and
// queries multiplied by it, so every q . k (hence the softmax) is kept while the spread
// between outlier channels and the others is square-rooted. An all-zero channel keeps
// norm 1.
//
// The statistics pass is HBM-bound (2 bytes read per element): workgroups of 4 waves each
// reduce 256 tokens of one row to 128 channel maxima (a lane owns 8 channels of one token,
// 16 lanes a token; 16 loads of 16 bytes in flight per lane), and merge them into the
// caller's norm buffer with one integer atomic max per channel. The maximum is taken over
// the fp16 magnitude bits (|x| as an unsigned 15-bit pattern orders like |x| for finite
// values), the buffer holding those bits until a last pass turns them into
// sqrt(float(|x|max)), or 1 for 0. Three launches, no memory beyond the caller's buffer.
//
// The scaling pass is an elementwise map, 2 bytes read and 2 written per element:
// y = fp16(x / norm) for keys, fp16(x * norm) for queries, one IEEE binary32 operation
// (division correctly rounded) then round to nearest even.
#include "kvq_device.h"
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kNormTokens = 256;    // tokens per workgroup of the statistics pass
constexpr int kNormSteps = kNormTokens / 16;
constexpr int kScaleTokens = 64;    // tokens per workgroup of the scaling pass
constexpr int kScaleSteps = kScaleTokens / 16;

__global__ __launch_bounds__(256) void norm_clear_kernel(uint32_t *__restrict__ m, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) m[i] = 0u;
}

__global__ __launch_bounds__(256) void norm_max_kernel(const uint16_t *__restrict__ src,
                                                       int64_t row_stride, int64_t tok_stride,
                                                       int32_t n_tokens, int32_t chunks,
                                                       uint32_t *__restrict__ m)
{
    __shared__ uint32_t red[4][kHeadDim];
    const int64_t row = blockIdx.x / chunks;
    const int chunk = (int)(blockIdx.x % chunks);
    const int oct = threadIdx.x & 15;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = chunk * kNormTokens + (threadIdx.x >> 4);
    const uint16_t *base = src + row * row_stride + oct * 8;

    u32x4 w[kNormSteps];
#pragma unroll
    for (int j = 0; j < kNormSteps; ++j) {
        const int t = t0 + 16 * j;
        w[j] = t < n_tokens ? *reinterpret_cast<const u32x4 *>(base + (int64_t)t * tok_stride)
                            : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[i] = 0u;
#pragma unroll
    for (int j = 0; j < kNormSteps; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mx[2 * k] = max(mx[2 * k], w[j][k] & 0x7fffu);
            mx[2 * k + 1] = max(mx[2 * k + 1], (w[j][k] >> 16) & 0x7fffu);
        }
    }
    // lanes l, l^16, l^32, l^48 of a wave hold the same channels
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx[i] = max(mx[i], (uint32_t)__shfl_xor((int)mx[i], 16));
        mx[i] = max(mx[i], (uint32_t)__shfl_xor((int)mx[i], 32));
    }
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][oct * 8 + i] = mx[i];
    }
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
        const int c = threadIdx.x;
        const uint32_t v = max(max(red[0][c], red[1][c]), max(red[2][c], red[3][c]));
        if (v != 0u) atomicMax(m + row * kHeadDim + c, v);
    }
}

__global__ __launch_bounds__(256) void norm_finish_kernel(uint32_t *__restrict__ m, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = m[i];
    const float mx = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    m[i] = __float_as_uint(bits == 0u ? 1.0f : __builtin_sqrtf(mx));
}

struct CSArgs {
    const uint16_t *x;
    int64_t x_row_stride, x_tok_stride;
    uint16_t *y;
    int64_t y_row_stride, y_tok_stride;
    const float *norm;
    int64_t rows_per_norm;
    int32_t n_tokens, chunks;
};

template <bool MULTIPLY>
__global__ __launch_bounds__(256) void channel_scale_kernel(CSArgs a)
{
    const int64_t row = blockIdx.x / a.chunks;
    const int chunk = (int)(blockIdx.x % a.chunks);
    const int oct = threadIdx.x & 15;
    const int t0 = chunk * kScaleTokens + (threadIdx.x >> 4);
    const float4_t *np =
        reinterpret_cast<const float4_t *>(a.norm + (row / a.rows_per_norm) * kHeadDim + oct * 8);
    const float4_t n0 = np[0], n1 = np[1];
    const float nv[8] = {n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3]};
    const uint16_t *xb = a.x + row * a.x_row_stride + oct * 8;
    uint16_t *yb = a.y + row * a.y_row_stride + oct * 8;

    u32x4 w[kScaleSteps];
#pragma unroll
    for (int j = 0; j < kScaleSteps; ++j) {
        const int t = t0 + 16 * j;
        w[j] = t < a.n_tokens ? *reinterpret_cast<const u32x4 *>(xb + (int64_t)t * a.x_tok_stride)
                              : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kScaleSteps; ++j) {
        const int t = t0 + 16 * j;
        if (t >= a.n_tokens) continue;
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const half2_t h = as_h2(w[j][k]);   // by value: a bit_cast of the element itself reads element 0
            const float x0 = (float)h.x, x1 = (float)h.y;
            float y0 = MULTIPLY ? x0 * nv[2 * k] : x0 / nv[2 * k];
            float y1 = MULTIPLY ? x1 * nv[2 * k + 1] : x1 / nv[2 * k + 1];
            // keep the binary32 result: without the barrier the product and the fp16
            // conversion may become one v_fma_mix (a single rounding to fp16)
            asm("" : "+v"(y0), "+v"(y1));
            o[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
        }
        *reinterpret_cast<u32x4 *>(yb + (int64_t)t * a.y_tok_stride) = o;
    }
}

}  // namespace

hipError_t launch_key_norm(const uint16_t *k, int64_t n_rows, int32_t n_tokens,
                           int64_t row_stride, int64_t tok_stride, float *norm,
                           hipStream_t stream)
{
    uint32_t *m = reinterpret_cast<uint32_t *>(norm);
    const int64_t n = n_rows * kHeadDim;
    const uint32_t fill_wg = (uint32_t)((n + 255) / 256);
    hipLaunchKernelGGL(norm_clear_kernel, dim3(fill_wg), dim3(256), 0, stream, m, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (n_tokens > 0) {
        const int32_t chunks = (n_tokens + kNormTokens - 1) / kNormTokens;
        hipLaunchKernelGGL(norm_max_kernel, dim3((uint32_t)(n_rows * chunks)), dim3(256), 0,
                           stream, k, row_stride, tok_stride, n_tokens, chunks, m);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(norm_finish_kernel, dim3(fill_wg), dim3(256), 0, stream, m, n);
    return hipGetLastError();
}

hipError_t launch_channel_scale(const uint16_t *x, int64_t n_rows, int32_t n_tokens,
                                int64_t x_row_stride, int64_t x_tok_stride, const float *norm,
                                int64_t rows_per_norm, int multiply, uint16_t *y,
                                int64_t y_row_stride, int64_t y_tok_stride, hipStream_t stream)
{
    if (n_tokens == 0) return hipSuccess;
    CSArgs a{x, x_row_stride, x_tok_stride, y, y_row_stride, y_tok_stride, norm, rows_per_norm,
             n_tokens, (n_tokens + kScaleTokens - 1) / kScaleTokens};
    const dim3 grid((uint32_t)(n_rows * a.chunks));
    if (multiply)
        hipLaunchKernelGGL(channel_scale_kernel<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(channel_scale_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
