// decode_valu.hip -- the split-K decode partials of kvq_decode_attention computed with VALU
// dot products only (v_dot2_f32_f16, no matrix cores). Same arguments and partial layout
// as the MFMA kernel in decode_attn.hip; it exists as the measured comparison for that
// design choice (exported as kvq_decode_attention_valu).
//
// What is computed is the same: for each query head, softmax(sm * q K^T) V over the split's
// packed tokens, dequantized as zero + code * scale (InnerQ page "KV缓存量化技术InnerQ：提升
// 大模型推理效率" sec. 3.1), plus the fp16 window tokens in the designated split
// (BitDecoding page "Tensor Core加速的低比特KV缓存解码系统" sec. 2.2).
//
// Mapping: one workgroup per (batch, kv-head, split, chunk of <= 4 query heads), 4 waves;
// wave w works on query head w of the chunk over every tile of the split. Tiles are staged
// in a 3-slot LDS ring shared by the workgroup (wave 0 issues the direct-to-LDS loads; a
// barrier publishes a tile and another frees its slot).
//  * Q K^T: lane (t, c) takes token t and the channel half c (groups 2c, 2c+1); the codes
//    enter v_dot2_f32_f16 as fp16 64 + code and the accumulator starts at -64 * sum(q over
//    the group), as in the MFMA kernel. The two halves are added across lanes t, t + 32.
//  * P V: lane j takes channels 2j, 2j+1 and runs over the tile's tokens in pairs: the
//    weights p * scale_v (fp16 high part + fp16 remainder) against the code pairs.
#include "decode_common.h"
#include "kvq_internal.h"

#include <math.h>

namespace kvq {
namespace {

constexpr int kVRing = 3;

template <int TILE_BYTES>
struct SmemV {
    alignas(16) uint8_t ring[kVRing][TILE_BYTES];
    alignas(16) uint16_t q[4][kHeadDim];
    alignas(16) float p[4][kTile];
};

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c)
{
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask)
{
    const int lane = threadIdx.x & 63;
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) * 4, __float_as_int(v)));
}

// the code field of channels 2j, 2j+1 of token t (channel 2j in the low BITS bits, 2j+1 in
// the next BITS bits), from the staged V code rows; for 3 bits the field may straddle two
// dwords (the second one exists: it is at most the first dword after the V code rows, in
// the same slot)
template <int BITS>
__device__ __forceinline__ uint32_t v_pair_bits(const uint8_t *vcodes, int t, int j)
{
    constexpr int TOKB = kHeadDim * BITS / 8;
    const int bit = 2 * BITS * j;
    const uint32_t *d = reinterpret_cast<const uint32_t *>(vcodes + t * TOKB + ((bit >> 5) << 2));
    if (BITS == 3) return __builtin_amdgcn_alignbit(d[1], d[0], bit & 31);
    return d[0] >> (bit & 31);
}

// one wave's online-softmax state for its head; lane j owns channels 2j, 2j+1
struct HeadState {
    float m, lsum;     // running max (exp2 domain); lane partial of sum p (lanes 0..31)
    float oe, oo, zt;  // sum_t w_t (64 + code) for channels 2j, 2j+1; sum_t p_t zero'_t
};

// softmax step for one tile: l = logits of token t (lanes t and t + 32 alike), big = any V
// scale of the tile large enough that p * scale could leave fp16 with p up to 2^kSlack
__device__ __forceinline__ float softmax_step(float l, bool big, int lane, HeadState &st)
{
    float tmax = row_max16(l);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    const bool grow = (tmax > st.m + kSlack) || (big && tmax > st.m);   // wave-uniform
    if (grow) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - tmax);
        st.m = tmax;
        st.lsum *= alpha;
        st.oe *= alpha;
        st.oo *= alpha;
        st.zt *= alpha;
    }
    const float p = __builtin_amdgcn_exp2f(l - st.m);
    if (lane < 32) st.lsum += p;
    return p;
}

// P V of one tile: p32 = the tile's p values (token order), sd[t] = {scale_v, zero_v} of
// token t for this lane's group (fp16 1.0 / 0 for window tokens), cb[t] = code field of the
// lane's two channels (packed tiles) -- or, for window tokens, the fp16 pair itself
template <int BITS, bool PACKED>
__device__ __forceinline__ void pv_pairs(const float p32[kTile], const uint32_t sd[kTile],
                                         const uint32_t cb[kTile], const Magic &M, HeadState &st)
{
    constexpr uint32_t mask = ((1u << BITS) - 1u) * 0x00100010u;   // code bits at 4.. of each half
#pragma unroll
    for (int u = 0; u < kTile / 2; ++u) {
        const float p0 = p32[2 * u], p1 = p32[2 * u + 1];
        const uint32_t hi = pv_hi(p0, sd[2 * u], p1, sd[2 * u + 1]);
        const uint32_t lo = pv_lo(p0, sd[2 * u], p1, sd[2 * u + 1], hi);
        half2_t be, bo;
        if (PACKED) {
            const uint32_t uc = pack_lo16(cb[2 * u], cb[2 * u + 1]);
            be = as_h2(mpair(uc << 4, mask, M.b6));
            bo = as_h2(mpair(BITS == 4 ? uc : uc << (4 - BITS), mask, M.b6));
            const half2_t z0 = as_h2(sd[2 * u]), z1 = as_h2(sd[2 * u + 1]);
            // the B operand carries codes + 64: zero' = zero - 64 * scale
            st.zt = __builtin_fmaf(p0, __builtin_fmaf(-64.0f, (float)z0.x, (float)z0.y), st.zt);
            st.zt = __builtin_fmaf(p1, __builtin_fmaf(-64.0f, (float)z1.x, (float)z1.y), st.zt);
        } else {
            be = as_h2(pack_lo16(cb[2 * u], cb[2 * u + 1]));
            bo = as_h2(pack_hi16(cb[2 * u], cb[2 * u + 1]));
        }
        st.oe = dot2(as_h2(hi), be, st.oe);
        st.oe = dot2(as_h2(lo), be, st.oe);
        st.oo = dot2(as_h2(hi), bo, st.oo);
        st.oo = dot2(as_h2(lo), bo, st.oo);
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecArgs a)
{
    using G = TileGeom<BITS>;
    __shared__ SmemV<G::BYTES> sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    const int split = blockIdx.y;
    const int b = (int)(row / a.Hkv);
    const int kvh = (int)(row % a.Hkv);
    const int h0 = kvh * a.gq + blockIdx.z * 4;
    const int nh = a.gq - (int)blockIdx.z * 4 < 4 ? a.gq - (int)blockIdx.z * 4 : 4;
    const bool live = wave < nh;

    int tlo, thi;
    bool with_res;
    split_range(a, split, tlo, thi, with_res);
    const int ntiles = thi - tlo;

    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.kp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.vp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q), 0, a.q_bytes, kRsrcWord3);

    // ---- wave 0: q of the chunk's 4 heads (1 KB), then the first two tiles ----
    if (wave == 0) {
        dma(rq, reinterpret_cast<uint8_t *>(&sm.q[0][0]),
            (uint32_t)(((int64_t)b * a.Hq + h0) * kHeadDim * 2) + lane * 16, 16);
#pragma unroll
        for (int k = 0; k < kVRing - 1; ++k)
            if (k < ntiles) issue_tile<BITS>(rk, rv, &sm.ring[k][0], tlo + k, lane, a.block_bytes, a.sz_off);
        wait_behind<BITS>(ntiles < kVRing - 1 ? ntiles : kVRing - 1);
    }
    __syncthreads();

    // ---- this wave's head: q octets of groups 2c, 2c+1 in the code slot order, sums ----
    const int t = lane & 31, c = lane >> 5;
    const int h = wave < 4 ? wave : 0;
    half8_t qo[2][4];
    float qs[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        float s = 0.0f;
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.q[h][32 * (2 * c + jj) + 8 * o]);
            qo[jj][o] = perm_octet_f16(w);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += (float)qo[jj][o][e];
        }
        qs[jj] = s;
    }
    const int j = lane, g = lane >> 4;     // P V: channels 2j, 2j+1 of group g
    const Magic M;
    HeadState st;
    st.m = -INFINITY;
    st.lsum = st.oe = st.oo = st.zt = 0.0f;

    // ---- packed tiles ----
    for (int k = 0; k < ntiles; ++k) {
        if (wave == 0) {
            if (k + kVRing - 1 < ntiles)
                issue_tile<BITS>(rk, rv, &sm.ring[(k + kVRing - 1) % kVRing][0], tlo + k + kVRing - 1,
                                 lane, a.block_bytes, a.sz_off);
            const int younger = ntiles - 1 - k < kVRing - 1 ? ntiles - 1 - k : kVRing - 1;
            wait_behind<BITS>(younger);
        }
        __syncthreads();                       // tile k is in LDS for every wave
        if (live) {
            const uint8_t *slot = &sm.ring[k % kVRing][0];
            // Q K^T for token t, groups 2c + jj
            float part = 0.0f;
            bool big = false;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                KGroup<BITS> kg;
                kg.load(slot, t, 2 * c + jj);
                float acc = -64.0f * qs[jj];
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const half8_t kv = kg.octet(o, M);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc = dot2(half2_t{qo[jj][o][2 * e], qo[jj][o][2 * e + 1]},
                                   half2_t{kv[2 * e], kv[2 * e + 1]}, acc);
                }
                const half2_t szk = as_h2(*reinterpret_cast<const uint32_t *>(
                    slot + G::KSZ + t * 16 + 4 * (2 * c + jj)));
                part = __builtin_fmaf((float)szk.x, acc, part);
                part = __builtin_fmaf((float)szk.y, qs[jj], part);
                const half2_t szv = as_h2(*reinterpret_cast<const uint32_t *>(
                    slot + G::VSZ + t * 16 + 4 * (2 * c + jj)));
                big |= szv.x >= (_Float16)kBigScale;
            }
            const float l = (part + shfl_xor_f(part, 32)) * a.sm_log2;
            const bool any_big = __builtin_amdgcn_ballot_w64(big) != 0;
            const float p = softmax_step(l, any_big, lane, st);
            if (lane < 32) sm.p[wave][t] = p;
            lds_fence();
            float p32[kTile];
            uint32_t sd[kTile], cb[kTile];
#pragma unroll
            for (int q4 = 0; q4 < kTile / 4; ++q4) {
                const float4_t v = *reinterpret_cast<const float4_t *>(&sm.p[wave][4 * q4]);
                p32[4 * q4] = v[0];
                p32[4 * q4 + 1] = v[1];
                p32[4 * q4 + 2] = v[2];
                p32[4 * q4 + 3] = v[3];
            }
#pragma unroll
            for (int tt = 0; tt < kTile; ++tt) {
                sd[tt] = *reinterpret_cast<const uint32_t *>(slot + G::VSZ + tt * 16 + 4 * g);
                cb[tt] = v_pair_bits<BITS>(slot + G::CB, tt, j);
            }
            pv_pairs<BITS, true>(p32, sd, cb, M, st);
        }
        __syncthreads();                       // slot k % 3 may be refilled
    }

    // ---- fp16 window tokens (designated split), 32 at a time, straight from memory ----
    if (with_res && live) {
        const uint16_t *kr = a.kres + row * a.res_cap * kHeadDim;
        const uint16_t *vr = a.vres + row * a.res_cap * kHeadDim;
        for (int rt = 0; rt * kTile < a.n_res; ++rt) {
            const int ts = rt * kTile + t;
            const int tc = ts < a.n_res ? ts : a.n_res - 1;
            float part = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float acc = 0.0f;
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const half8_t kv = perm_octet_f16(*reinterpret_cast<const u32x4 *>(
                        kr + (int64_t)tc * kHeadDim + 32 * (2 * c + jj) + 8 * o));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc = dot2(half2_t{qo[jj][o][2 * e], qo[jj][o][2 * e + 1]},
                                   half2_t{kv[2 * e], kv[2 * e + 1]}, acc);
                }
                part += acc;
            }
            const float tot = part + shfl_xor_f(part, 32);
            const float l = ts < a.n_res ? tot * a.sm_log2 : -INFINITY;
            const float p = softmax_step(l, false, lane, st);
            if (lane < 32) sm.p[wave][t] = p;
            lds_fence();
            float p32[kTile];
            uint32_t sd[kTile], cb[kTile];
#pragma unroll
            for (int tt = 0; tt < kTile; ++tt) {
                p32[tt] = sm.p[wave][tt];
                const int tr = rt * kTile + tt < a.n_res ? rt * kTile + tt : a.n_res - 1;
                sd[tt] = 0x3C00u;              // scale 1, zero 0
                cb[tt] = *reinterpret_cast<const uint32_t *>(vr + (int64_t)tr * kHeadDim + 2 * j);
            }
            pv_pairs<BITS, false>(p32, sd, cb, M, st);
            lds_fence();                       // p read before the next window tile rewrites it
        }
    }

    // ---- this head's partial ----
    if (live) {
        float L = row_sum16(st.lsum);
        L += shfl_xor_f(L, 16);
        L += shfl_xor_f(L, 32);
        const int64_t hq = (int64_t)b * a.Hq + h0 + wave;
        const int64_t ob = (hq * a.S + split) * kHeadDim + 2 * j;
        float v0 = 0.f, v1 = 0.f, lse = -INFINITY;
        if (L > 0.f) {
            const float inv = 1.0f / L;
            v0 = (st.oe + st.zt) * inv;
            v1 = (st.oo + st.zt) * inv;
            lse = (st.m + __log2f(L)) * 0.69314718055994531f;
        }
        a.part_o[ob] = v0;
        a.part_o[ob + 1] = v1;
        if (lane == 0) a.part_lse[hq * a.S + split] = lse;
    }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams &p, hipStream_t stream)
{
    DecArgs a = make_dec_args(p);
    a.head_base = 0;
    const int64_t rows = (int64_t)p.B * p.Hkv;
    const int chunks = (a.gq + 3) / 4;
    const dim3 grid((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks);
    switch (p.bits) {
    case 2: hipLaunchKernelGGL(decode_valu_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(decode_valu_kernel<3>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_valu_kernel<4>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
