// paged.hip -- token-wise packing into a paged cache and the per-token sliding window.
//
// InnerQ page ("KV缓存量化技术InnerQ：提升大模型推理效率") sec. 2.3: a new token always enters
// the fp16 recent window; once the window is full its oldest token is quantized into the
// main cache; the sink window, filled at prefill, never changes. 3-bit blog page
// ("3-bit KV缓存量化：大模型推理功耗与带宽优化核心技术") sec. 6.1: the packed cache lives in
// pages of a byte pool reached through a per-sequence block table. Because the groups run
// along head_dim, a token's codes depend on that token only, so one token at a time can be
// packed into its slot of a block without touching its neighbours.
//
// Packed token j of sequence b, kv-head h: pool block tbl[b][j / 128] at
// pool + blk * block_stride + h * head_stride, token j % 128 inside the block. A table
// entry outside [0, pool_blocks) or a position beyond the table is skipped (nothing is
// written), so a wrong table can give wrong results but never an access outside the pool.
#include <type_traits>

#include "kvq_internal.h"
#include "paged_common.h"
#include "quant_common.h"

namespace kvq {
namespace {

constexpr int kPackTokens = 64;          // tokens per workgroup of the token packer

struct PackArgs {
    const uint16_t *src;
    int64_t src_row_stride, src_tok_stride;
    const int32_t *count, *start;
    int32_t Hkv, chunks, max_count;
    PoolGeom g;
};

// One workgroup per (row, 64 source tokens): 16 lanes per token, 16 tokens per pass.
template <int BITS, bool HYBRID>
__global__ __launch_bounds__(256) void pack_tokens_kernel(PackArgs a)
{
    const int64_t row = blockIdx.x / a.chunks;
    const int chunk = (int)(blockIdx.x % a.chunks);
    const int b = (int)(row / a.Hkv), h = (int)(row % a.Hkv);
    int cnt = __builtin_amdgcn_readfirstlane(a.count[b]);
    cnt = cnt < a.max_count ? cnt : a.max_count;          // the source holds max_count tokens
    const int st0 = __builtin_amdgcn_readfirstlane(a.start[b]);
    const int oct = threadIdx.x & 15;
    const int tl = threadIdx.x >> 4;
    const uint16_t *src = a.src + row * a.src_row_stride + oct * 8;

    u32x4 raw[kPackTokens / 16];
#pragma unroll
    for (int p = 0; p < kPackTokens / 16; ++p) {
        const int t = chunk * kPackTokens + p * 16 + tl;
        raw[p] = t < cnt ? *reinterpret_cast<const u32x4 *>(src + (int64_t)t * a.src_tok_stride)
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < kPackTokens / 16; ++p) {
        const int t = chunk * kPackTokens + p * 16 + tl;
        if (t >= cnt) continue;                 // a whole token (16 lanes, 4 quads) at a time
        uint32_t packed;
        uint16_t s, z;
        int flag;
        quantize_octet<BITS, HYBRID>(raw[p], packed, s, z, flag);
        const int64_t j = (int64_t)st0 + t;
        uint8_t *blk = block_of(a.g, b, h, j);
        if (blk) store_octet<BITS, HYBRID>(blk, a.g, (int)(j & 127), oct, packed, s, z, flag);
    }
}

struct EvictArgs {
    const uint16_t *k_new, *v_new;
    uint16_t *k_res, *v_res;
    int32_t res_cap, n_sink, Hkv;
    int32_t *state;                      // [B][4]: n_packed, n_res, next_slot, unused
    PoolGeom kg, vg;
};

// One workgroup per sequence: 16 lanes per (kv-head, K or V) token, 16 tokens per pass.
// Each lane reads the slot's old 16 bytes (to evict them) before it writes the new token's
// 16 bytes into the same place; the state is updated once every lane is done.
template <int BITS, bool HYBRID>
__global__ __launch_bounds__(256) void append_evict_kernel(EvictArgs a)
{
    const int b = blockIdx.x;
    // (plain loads: this kernel writes the state back at the end)
    const int4 st = *reinterpret_cast<const int4 *>(a.state + 4 * (int64_t)b);
    const int n_packed = __builtin_amdgcn_readfirstlane(st.x);
    const int n_res = __builtin_amdgcn_readfirstlane(st.y);
    const int nxt = __builtin_amdgcn_readfirstlane(st.z);
    const int pad = st.w;
    const bool full = n_res >= a.res_cap;
    // a state outside its range is brought back into it (never an access outside the window)
    int slot = full ? nxt : (n_res < 0 ? 0 : n_res);
    if (full && (slot < a.n_sink || slot >= a.res_cap)) slot = a.n_sink;
    const int oct = threadIdx.x & 15;
    const int tl = threadIdx.x >> 4;
    const int items = 2 * a.Hkv;
    for (int it0 = 0; it0 < items; it0 += 16) {
        const int item = it0 + tl;
        if (item >= items) continue;
        const int h = item >> 1;
        const bool is_v = item & 1;
        const int64_t wrow = (int64_t)b * a.Hkv + h;
        uint16_t *win = (is_v ? a.v_res : a.k_res) + (wrow * a.res_cap + slot) * kHeadDim + oct * 8;
        const u32x4 nw = *reinterpret_cast<const u32x4 *>((is_v ? a.v_new : a.k_new) +
                                                          wrow * kHeadDim + oct * 8);
        if (full) {
            const u32x4 old = *reinterpret_cast<const u32x4 *>(win);
            uint32_t packed;
            uint16_t s, z;
            int flag;
            quantize_octet<BITS, HYBRID>(old, packed, s, z, flag);
            const PoolGeom &g = is_v ? a.vg : a.kg;
            uint8_t *blk = block_of(g, b, h, n_packed);
            if (blk) store_octet<BITS, HYBRID>(blk, g, n_packed & 127, oct, packed, s, z, flag);
        }
        *reinterpret_cast<u32x4 *>(win) = nw;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int4 ns;
        if (full) {
            ns.x = n_packed + 1;
            ns.y = a.res_cap;
            ns.z = slot + 1 < a.res_cap ? slot + 1 : a.n_sink;
        } else {
            ns.x = n_packed;
            ns.y = slot + 1;
            ns.z = nxt;
        }
        ns.w = pad;
        *reinterpret_cast<int4 *>(a.state + 4 * (int64_t)b) = ns;
    }
}

template <bool HYBRID, class F>
hipError_t by_bits(int bits, F &&f)
{
    switch (bits) {
    case 2: return f(std::integral_constant<int, 2>{}, std::integral_constant<bool, HYBRID>{});
    case 3: return f(std::integral_constant<int, 3>{}, std::integral_constant<bool, HYBRID>{});
    case 4: return f(std::integral_constant<int, 4>{}, std::integral_constant<bool, HYBRID>{});
    default: return hipErrorInvalidValue;
    }
}

template <class F>
hipError_t dispatch(int bits, int hybrid, F &&f)
{
    return hybrid ? by_bits<true>(bits, f) : by_bits<false>(bits, f);
}

}  // namespace

hipError_t launch_pack_tokens_paged(const PagedPool &pool, const uint16_t *src, int32_t B,
                                    int32_t Hkv, int64_t src_row_stride, int64_t src_tok_stride,
                                    const int32_t *count, const int32_t *start, int32_t max_count,
                                    uint8_t *dst_pool, hipStream_t stream)
{
    if (max_count <= 0) return hipSuccess;
    PackArgs a{src, src_row_stride, src_tok_stride, count, start, Hkv,
               (max_count + kPackTokens - 1) / kPackTokens, max_count,
               PoolGeom{dst_pool, pool.pool_blocks, pool.block_stride, pool.head_stride, pool.tbl,
                        pool.max_blocks, pool.sz_off, pool.flag_off}};
    const dim3 grid((uint32_t)((int64_t)B * Hkv * a.chunks));
    return dispatch(pool.bits, pool.hybrid, [&](auto bits, auto hyb) {
        hipLaunchKernelGGL((pack_tokens_kernel<decltype(bits)::value, decltype(hyb)::value>), grid,
                           dim3(256), 0, stream, a);
        return hipGetLastError();
    });
}

hipError_t launch_copy_state(int32_t *dst, const int32_t *src, int32_t B, hipStream_t stream)
{
    return hipMemcpyAsync(dst, src, (size_t)B * 4 * sizeof(int32_t), hipMemcpyDeviceToDevice,
                          stream);
}

hipError_t launch_append_evict(const PagedPool &pool, const uint16_t *k_new,
                               const uint16_t *v_new, uint16_t *k_res, uint16_t *v_res,
                               int32_t res_cap, int32_t n_sink, uint8_t *k_pool, uint8_t *v_pool,
                               int32_t *state, int32_t B, int32_t Hkv, hipStream_t stream)
{
    const PoolGeom kg{k_pool, pool.pool_blocks, pool.block_stride, pool.head_stride, pool.tbl,
                      pool.max_blocks, pool.sz_off, pool.flag_off};
    PoolGeom vg = kg;
    vg.pool = v_pool;
    EvictArgs a{k_new, v_new, k_res, v_res, res_cap, n_sink, Hkv, state, kg, vg};
    return dispatch(pool.bits, pool.hybrid, [&](auto bits, auto hyb) {
        hipLaunchKernelGGL((append_evict_kernel<decltype(bits)::value, decltype(hyb)::value>),
                           dim3((uint32_t)B), dim3(256), 0, stream, a);
        return hipGetLastError();
    });
}

}  // namespace kvq
