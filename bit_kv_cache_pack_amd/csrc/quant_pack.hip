// quant_pack.hip -- group-wise low-bit quantization of fp16 K/V tokens into packed blocks.
//
// Follows the BitDecoding page ("Tensor Core加速的低比特KV缓存解码系统") sec. 2.1 for
// scale = (max - min) / (2^b - 1) and code = round((x - min) / scale), and sec. 3.1 for the
// register-only kernel shape (per-thread min/max, a cross-lane reduction, packing in
// registers); the 3-bit blog page ("3-bit KV缓存量化：大模型推理功耗与带宽优化核心技术")
// sec. 2.3 for the clip to [0, 2^b - 1] and sec. 3.2 for fp16 K/V -> packed codes +
// scale/zero; the InnerQ page ("KV缓存量化技术InnerQ：提升大模型推理效率") sec. 2.1 for
// groups of 32 along head_dim and sec. 2.2 for the per-group symmetric/asymmetric choice.
//
// Work mapping: one workgroup (4 waves) per (row, 128-token block). A lane owns 8
// channels (one 16-byte load); 4 lanes (a DPP quad) hold one 32-channel group, 16 lanes
// one token, so a wave covers 4 tokens per step and 32 tokens in all. The group min/max
// and the hybrid error sums are quad reductions with DPP; a lane's 8 codes are exactly
// `bits` bytes of the group's word, so every lane stores its own bytes.
//
// The scales are IEEE binary32 operations (no contraction: see the pragma; division is
// the correctly rounded one) and each code is the one the correctly rounded quotient
// gives (taken from a reciprocal where that is provably the same, see quant_common.h), so
// the bytes equal the CPU definition's.
#include "kvq_internal.h"
#include "quant_common.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

struct QPArgs {
    const uint16_t *src;
    int64_t src_row_stride, src_tok_stride;  // elements
    uint8_t *dst;
    int64_t dst_row_stride;                  // bytes
    int32_t first_block, n_blocks;
    int32_t block_bytes, sz_off, flag_off;
};

template <int BITS, bool HYBRID>
__global__ __launch_bounds__(256) void quant_pack_kernel(QPArgs a)
{
    constexpr int GBYTES = 4 * BITS;   // bytes per packed group

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row = blockIdx.x / a.n_blocks;
    const int blk = blockIdx.x % a.n_blocks;
    const int tl = lane >> 4;          // token within a 4-token step
    const int oct = lane & 15;         // channel octet 0..15
    const int g = oct >> 2;            // group 0..3
    const int j = oct & 3;             // octet within the group

    // hybrid mode flags of this wave's 32 tokens: bits wave*128 .. wave*128+127 of the
    // block's 512 (bit = token * 4 + group), gathered from wave ballots, no LDS
    uint32_t fw[4] = {0u, 0u, 0u, 0u};

    const uint16_t *src = a.src + row * a.src_row_stride + (int64_t)blk * kBlockTokens * a.src_tok_stride;
    uint8_t *dblk = a.dst + row * a.dst_row_stride + (int64_t)(a.first_block + blk) * a.block_bytes;

    // issue all 8 loads of this wave's 32 tokens first
    u32x4 raw[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tb = wave * 32 + it * 4 + tl;
        raw[it] = *reinterpret_cast<const u32x4 *>(src + (int64_t)tb * a.src_tok_stride + oct * 8);
    }

#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tb = wave * 32 + it * 4 + tl;
        uint32_t packed;
        uint16_t out_s, out_z;
        int flag;
        quantize_octet<BITS, HYBRID>(raw[it], packed, out_s, out_z, flag);

        uint8_t *gptr = dblk + (tb * kGroups + g) * GBYTES + j * BITS;
        if (BITS == 4) {
            *reinterpret_cast<uint32_t *>(gptr) = packed;
        } else if (BITS == 2) {
            *reinterpret_cast<uint16_t *>(gptr) = (uint16_t)packed;
        } else {
            gptr[0] = (uint8_t)packed;
            gptr[1] = (uint8_t)(packed >> 8);
            gptr[2] = (uint8_t)(packed >> 16);
        }
        if (j == 0)
            *reinterpret_cast<uint32_t *>(dblk + a.sz_off + (tb * kGroups + g) * 4) =
                (uint32_t)out_s | ((uint32_t)out_z << 16);
        if (HYBRID) {
            // lane 16 tl + 4 g holds the flag of token tl, group g of this step: its bit is
            // it * 16 + tl * 4 + g of the wave's range
            const uint64_t m = __builtin_amdgcn_ballot_w64(j == 0 && flag);
            uint32_t b16 = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) b16 |= (uint32_t)((m >> (16 * (k >> 2) + 4 * (k & 3))) & 1u) << k;
            fw[it >> 1] |= b16 << (16 * (it & 1));
        }
    }
    if (HYBRID) {
        if (lane < 4)
            reinterpret_cast<uint32_t *>(dblk + a.flag_off)[wave * 4 + lane] =
                lane == 0 ? fw[0] : lane == 1 ? fw[1] : lane == 2 ? fw[2] : fw[3];
    }
}

template <int BITS, bool HYBRID>
hipError_t launch_t(const QPArgs &a, int64_t n_rows, hipStream_t stream)
{
    const int64_t n_wg = n_rows * a.n_blocks;
    hipLaunchKernelGGL((quant_pack_kernel<BITS, HYBRID>), dim3((uint32_t)n_wg), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack(int bits, int hybrid, const uint16_t *src, int64_t n_rows,
                                int32_t n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                                uint8_t *dst, int64_t dst_row_stride, int32_t first_block,
                                int32_t block_bytes, int32_t sz_off, int32_t flag_off,
                                hipStream_t stream)
{
    QPArgs a{src, src_row_stride, src_tok_stride, dst, dst_row_stride, first_block,
             n_tokens / kBlockTokens, block_bytes, sz_off, flag_off};
    switch (bits * 2 + (hybrid ? 1 : 0)) {
    case 4: return launch_t<2, false>(a, n_rows, stream);
    case 5: return launch_t<2, true>(a, n_rows, stream);
    case 6: return launch_t<3, false>(a, n_rows, stream);
    case 7: return launch_t<3, true>(a, n_rows, stream);
    case 8: return launch_t<4, false>(a, n_rows, stream);
    case 9: return launch_t<4, true>(a, n_rows, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
