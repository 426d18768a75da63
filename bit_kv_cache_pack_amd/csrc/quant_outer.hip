// quant_outer.hip -- outer-dimension (KIVI-style) group quantization, the grouping the
// InnerQ page ("KV缓存量化技术InnerQ：提升大模型推理效率") compares its own against (sec. 1:
// groups run along the sequence, so one token row mixes many groups; sec. 4.1 times it).
// A group is the 32 consecutive tokens 32*tg .. 32*tg+31 of one channel within a 128-token
// block; the quantizer is the asymmetric one of quant_common.h (min/max over the group,
// scale = fp16((max - min) / (2^b - 1)), zero = fp16(min), round half away, clip). Codes
// keep the inner layout's positions (token-major, LSB-first 32-channel words), so a decode
// reads them the same way; the scale/zero region holds [4 token groups][128 channels].
//
// One workgroup per (row, block): the 128 x 128 fp16 block is staged in LDS; a DPP quad
// takes one (token group, channel) group, a lane 8 of its tokens (read down a column of
// the staged block), and the codes go back to LDS as bytes; a second pass packs each
// token's 32-channel words.
#include "kvq_internal.h"
#include "quant_common.h"

namespace kvq {
namespace {

constexpr int kRowPad = 8;                                   // halves of padding per token row
constexpr int kLdsRow = kHeadDim + kRowPad;

struct QOArgs {
    const uint16_t *src;
    int64_t src_row_stride, src_tok_stride;
    uint8_t *dst;
    int64_t dst_row_stride;
    int32_t first_block, n_blocks;
    int32_t block_bytes, sz_off;
};

template <int BITS>
__global__ __launch_bounds__(256) void quant_outer_kernel(QOArgs a)
{
    constexpr int GBYTES = 4 * BITS;
    __shared__ uint16_t xs[kBlockTokens][kLdsRow];
    __shared__ uint8_t cs[kBlockTokens][kHeadDim];
    const int64_t row = blockIdx.x / a.n_blocks;
    const int blk = blockIdx.x % a.n_blocks;
    const uint16_t *src = a.src + row * a.src_row_stride + (int64_t)blk * kBlockTokens * a.src_tok_stride;
    uint8_t *dblk = a.dst + row * a.dst_row_stride + (int64_t)(a.first_block + blk) * a.block_bytes;

    // stage the block: 16 lanes per token row, 16 rows per pass
    {
        const int oct = threadIdx.x & 15;
        for (int t = threadIdx.x >> 4; t < kBlockTokens; t += 16)
            *reinterpret_cast<u32x4 *>(&xs[t][oct * 8]) =
                *reinterpret_cast<const u32x4 *>(src + (int64_t)t * a.src_tok_stride + oct * 8);
    }
    __syncthreads();

    // 512 groups, 64 quads per pass: group (tg, c), lane j of the quad holds tokens
    // 32 tg + 8 j .. +7 of channel c
    const int quad = threadIdx.x >> 2, j = threadIdx.x & 3;
#pragma unroll 1
    for (int p = 0; p < 8; ++p) {
        const int gid = p * 64 + quad;
        const int tg = gid >> 7, c = gid & 127;
        const int t0 = 32 * tg + 8 * j;
        u32x4 raw;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            raw[k] = (uint32_t)xs[t0 + 2 * k][c] | ((uint32_t)xs[t0 + 2 * k + 1][c] << 16);
        uint32_t packed;
        uint16_t s, z;
        int flag;
        quantize_octet<BITS, false>(raw, packed, s, z, flag);
#pragma unroll
        for (int i = 0; i < 8; ++i) cs[t0 + i][c] = (uint8_t)((packed >> (BITS * i)) & ((1u << BITS) - 1));
        if (j == 0)
            *reinterpret_cast<uint32_t *>(dblk + a.sz_off + (tg * kHeadDim + c) * 4) =
                (uint32_t)s | ((uint32_t)z << 16);
    }
    __syncthreads();

    // pack each token's four 32-channel words (LSB-first): 512 words, 2 per thread
#pragma unroll 1
    for (int w = threadIdx.x; w < kBlockTokens * kGroups; w += 256) {
        const int t = w >> 2, g = w & 3;
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t code = cs[t][32 * g + i];
            const int bit = BITS * i;
            word[bit >> 5] |= code << (bit & 31);
            if ((bit & 31) + BITS > 32) word[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }
        uint32_t *gp = reinterpret_cast<uint32_t *>(dblk + (t * kGroups + g) * GBYTES);
#pragma unroll
        for (int k = 0; k < BITS; ++k) gp[k] = word[k];
    }
}

template <int BITS>
hipError_t launch_t(const QOArgs &a, int64_t n_rows, hipStream_t stream)
{
    hipLaunchKernelGGL((quant_outer_kernel<BITS>), dim3((uint32_t)(n_rows * a.n_blocks)), dim3(256),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack_outer(int bits, const uint16_t *src, int64_t n_rows,
                                      int32_t n_tokens, int64_t src_row_stride,
                                      int64_t src_tok_stride, uint8_t *dst, int64_t dst_row_stride,
                                      int32_t first_block, int32_t block_bytes, int32_t sz_off,
                                      hipStream_t stream)
{
    QOArgs a{src, src_row_stride, src_tok_stride, dst, dst_row_stride, first_block,
             n_tokens / kBlockTokens, block_bytes, sz_off};
    switch (bits) {
    case 2: return launch_t<2>(a, n_rows, stream);
    case 3: return launch_t<3>(a, n_rows, stream);
    case 4: return launch_t<4>(a, n_rows, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
