// decode_attn.hip -- split-K decode attention straight from the packed low-bit cache.
//
// What is computed: for each query head, softmax(sm * q K^T) V over the split's packed
// tokens (dequantized as zero + code * scale, InnerQ page "KV缓存量化技术InnerQ：提升大模型推理
// 效率" sec. 3.1) and, for the designated split, the fp16 residual / sink tokens
// (BitDecoding page "Tensor Core加速的低比特KV缓存解码系统" sec. 2.2; InnerQ sec. 2.3).
// The query rows of one GQA group are processed together (BitDecoding sec. 2.3). Each
// split writes its normalised output and log-sum-exp; kvq_combine merges the splits.
//
// Mapping onto CDNA4 (our design; the pages' Tensor-Core / ldmatrix layouts are for other
// hardware):
//  * one workgroup = (batch, kv-head, split, head chunk of <= 4 query heads), 4 waves;
//    each wave streams 32-token tiles of the split (round robin) and keeps its own
//    online-softmax state; the waves are merged through LDS at the end.
//  * tiles reach LDS by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds) into a
//    two-slot ring per wave: a wave asks for its first two tiles up front and for tile k+2
//    once tile k is consumed, so ~10 KB per wave is in flight without holding it in VGPRs;
//    the wave waits on vmcnt for exactly the tile it is about to use.
//  * Q K^T uses v_mfma_f32_16x16x32_f16 with B = the integer codes as fp16 subnormals
//    (a code masked into mantissa bits k.. of a zero-exponent half is exactly
//    code * 2^(k-24); one AND per pair of codes) and rows i = 4*head + group of A holding
//    the query restricted to one 32-channel group, each channel divided by the power of
//    two its code slot carries. Lane (token n, r) loads group r of token n (one
//    16/12/8-byte load), and MFMA o consumes that group's channel octet o, so the result
//    row 4h+g is 2^-24 times head h's dot product with group g's codes. Every lane then
//    holds the four group dots of one (token, head) and applies its token's scale/zero:
//        l = sum_g scale_g * dot_g + zero_g * sum(q over g)
//    with no cross-lane reduction.
//  * P V uses the same MFMA with rows i = 4*head + group holding p * scale_v (split into
//    an fp16 high part and an fp16 remainder, two MFMAs, so the weights keep ~22 bits)
//    and B = the V codes (again subnormals) of 8 tokens x 1 channel per lane, built from
//    two tokens' code words at a time; each accumulator column is one channel, so its
//    power-of-two weight is divided out once after the last tile. Only rows whose group
//    matches the column's group are used; the zero-point term sum_t p_t zero_v is
//    accumulated on the VALU.
//    (The outer-grouped variant keeps codes + 64 from the fp16 magic-number trick.)
//  * row (16-lane) max / sum reductions use DPP; p passes through a 512 B per-wave LDS
//    slice to reach the PV operand layout, and the V scales are read straight from the
//    staged tile.
#include "decode_common.h"
#include "kvq.h"
#include "kvq_internal.h"
#include "paged_common.h"
#include "quant_common.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace kvq {
namespace {


// LDS of one workgroup: a RING-slot ring of tiles per wave plus small staging arrays
// (4-bit: ~49 KB with 2 slots, three workgroups per CU).
// A wave's merge output (mo) reuses the start of its own ring once its tiles are done.
template <int TILE_BYTES, int RING, int W, int QCOPIES = W>
struct Smem {
    alignas(16) uint8_t ring[W][RING][TILE_BYTES];    // per-wave ring of staged tiles
    alignas(16) uint16_t q[QCOPIES][4][kHeadDim];      // the chunk's q (one copy, or one per wave)
    alignas(16) float qn[kHeadDim];                    // the row's key-channel norms (if any)
    alignas(16) float p[W][2][4][kTile];      // p of head h, token t of tiles 2j and 2j+1
    alignas(16) float ml[W][4][2];
    // paged update: K and V of the token leaving the window ([0], [1]) and of the new one ([2], [3])
    alignas(16) uint16_t ev[4][kHeadDim];
    uint32_t evc[2][16], evs[2][4];           // its code words and scale/zero words
    uint32_t flag;                            // last-arrival flag of the fused split merge
    __device__ __forceinline__ float *mo(int w) { return reinterpret_cast<float *>(&ring[w][0][0]); }
};

template <int BITS>
__device__ __forceinline__ void pair_tokens(uint32_t a, uint32_t b, const Magic &M, half2_t out[8])
{
    if (BITS == 4) pair_tokens4(a, b, M, out);
    else if (BITS == 2) pair_tokens2(a, b, M, out);
    else pair_tokens3(a, b, M, out);
}

// PV operand slot order: slot e of lane group r holds tile token 4e + r, so the eight V-code
// reads of the four lane groups hit adjacent token rows (distinct LDS banks). Per-token
// values (p, scale_v) are stored at the slot position pos(t) = 8 * (t % 4) + t / 4 so that
// lane group r reads its eight values as two contiguous 16-byte words.
__device__ __forceinline__ int slot_pos(int t) { return 8 * (t & 3) + (t >> 2); }
// Position of token t's p in row h of a wave's p buffer. Odd rows swap the two 4-float
// halves of every 8-float block: the slots of tokens 0..15 (and those of 16..31) then sit
// on different banks in rows 2i and 2i+1, so neither the 32-lane stores of p nor the
// 16-byte reads of load_p8 meet a bank conflict (measured with the LDS counters).
__device__ __forceinline__ int p_pos(int h, int t) { return h * kTile + (slot_pos(t) ^ (4 * (h & 1))); }

// The packed kernel's q in LDS, as 64 pieces of 16 bytes (8 channels): channels
// 32 r + 8 o .. +7 of head h sit in piece 32 (o / 2) + 8 h + 2 r + o % 2. For one o the
// 16 pieces the lanes (head h, group r) read then lie as the p reads of load_p8 do, with
// no bank conflict (the plain head-major order has four-way conflicts there).
__device__ __forceinline__ int q_piece(int h, int r, int o) { return 32 * (o >> 1) + 8 * h + 2 * r + (o & 1); }
// the head-major piece (16 h + 4 r + o) that piece p of the LDS order holds
__device__ __forceinline__ int q_piece_src(int p)
{
    return 16 * ((p & 31) >> 3) + 4 * ((p & 7) >> 1) + 2 * (p >> 5) + (p & 1);
}

// v[k] for a lane-varying k in 0..3, as two levels of selects (a runtime vector index
// would otherwise go through scratch memory)
__device__ __forceinline__ float sel4(float4_t v, int k)
{
    const float a = (k & 1) ? v[1] : v[0];
    const float b = (k & 1) ? v[3] : v[2];
    return (k & 2) ? b : a;
}

// Online-softmax state of one wave: lane (n, r) tracks head r.
struct WaveState {
    float m, l;
    float zacc[4];     // sum_t p_t * zero_v(t, g) for head r, group g (lane partial)
    float4_t dpv[8];   // PV accumulators: rows 4h+g, column n <-> channel 8n + c
};

// Stage A of a tile leaves these for stage B (per lane): the V code words of channel
// octet n of tokens 4e + r, and the {scale_v, zero_v} dwords of tokens 4e + r, group gA
// (the A-operand row of this lane).
struct PVIn {
    uint32_t vc[8];
    uint32_t sd[8];
};

// The same for outer-grouped blocks: V codes as above, the {scale_v, zero_v} of channels
// 8n .. 8n+7 for the tile's token group, and the tile's sum of p for head r.
struct PVInO {
    uint32_t vc[8];
    uint32_t sz[8];
    float P;
};

// Online-softmax step of stage A for one tile. lg[u]: logits (exp2 domain) of token 16u + n
// for head r; zv[u][g]: V zero-point term of that token. Updates m, l and the zero-point
// sums, returns the tile's p values, and leaves the factor the PV accumulators must be
// multiplied by (once the previous tile's PV is in) in `alpha` when `rescale` is set.
__device__ __forceinline__ void softmax_a(const float lg[2], const float zv[2][4], bool big_scale,
                                          WaveState &st, float &p0, float &p1, float &alpha,
                                          bool &rescale)
{
    // Lazy rescale: the reference max m only moves when the tile's max exceeds it by more
    // than 2^kSlack (log2 units), or exceeds it at all while a V scale is so large that
    // p * scale could leave the fp16 range of the PV operand; otherwise p <= 2^kSlack.
    const float tmax = row_max16(fmaxf(lg[0], lg[1]));
    const bool grow = (tmax > st.m + kSlack) || (big_scale && tmax > st.m);
    rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
    alpha = 1.0f;
    if (rescale) {   // wave-uniform and rare once m has settled; alpha = 1 in every other lane
        const float mnew = grow ? tmax : st.m;
        alpha = grow ? __builtin_amdgcn_exp2f(st.m - mnew) : 1.0f;
        st.m = mnew;
        st.l *= alpha;
#pragma unroll
        for (int g = 0; g < 4; ++g) st.zacc[g] *= alpha;
    }
    p0 = __builtin_amdgcn_exp2f(lg[0] - st.m);
    p1 = __builtin_amdgcn_exp2f(lg[1] - st.m);
    st.l += p0 + p1;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.zacc[g] = __builtin_fmaf(p1, zv[1][g], __builtin_fmaf(p0, zv[0][g], st.zacc[g]));
}

// this lane's eight p values for stage B: head hA, token slots 8r .. 8r+7 (tokens 4e + r)
__device__ __forceinline__ void load_p8(const float *pw, int n, int r, float p8[8])
{
    const int hA = n >> 2;
    const int sw = 4 * (hA & 1);     // the half swap of odd rows (p_pos)
    const float4_t pl = *reinterpret_cast<const float4_t *>(pw + hA * kTile + 8 * r + sw);
    const float4_t ph = *reinterpret_cast<const float4_t *>(pw + hA * kTile + 8 * r + (4 - sw));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        p8[e] = pl[e];
        p8[4 + e] = ph[e];
    }
}

// Stage B core: PV for one tile. A operand: lane (i, r) holds rows i = 4h + g, token
// slots 8r .. 8r+7, i.e. tokens 4e + r; the weight p * scale_v is split into an fp16 high
// part and the fp16 of the remainder. vpair[m][c]: the V operand pair (slots 2m, 2m+1 of
// lane group r, i.e. tokens 8m + r and 8m + 4 + r; channel 8n + c). (Rows of heads beyond
// the chunk carry finite junk; their outputs are never stored.)
__device__ __forceinline__ void pv_mfma(const float p8[8], const uint32_t sd[8],
                                        const half2_t vpair[4][8], WaveState &st)
{
    u32x4 ahi, alo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ahi[k] = pv_hi(p8[2 * k], sd[2 * k], p8[2 * k + 1], sd[2 * k + 1]);
        alo[k] = pv_lo(p8[2 * k], sd[2 * k], p8[2 * k + 1], sd[2 * k + 1], ahi[k]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const half8_t bv{vpair[0][c].x, vpair[0][c].y, vpair[1][c].x, vpair[1][c].y,
                         vpair[2][c].x, vpair[2][c].y, vpair[3][c].x, vpair[3][c].y};
        st.dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ahi), bv,
                                                           st.dpv[c], 0, 0, 0);
        st.dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, alo), bv,
                                                           st.dpv[c], 0, 0, 0);
    }
}

template <int BITS>
__device__ __forceinline__ void raw_pair(uint32_t a, uint32_t b, half2_t out[8])
{
    if (BITS == 4) raw_pair4(a, b, out);
    else if (BITS == 2) raw_pair2(a, b, out);
    else raw_pair3(a, b, out);
}

// Stage B of a packed tile: the V codes enter as subnormals, so dpv[c] collects
// 2^(raw_value_shift(c) - 24) * sum_t p_t scale_t code_t (undone after the last tile).
template <int BITS>
__device__ __forceinline__ void stage_b_packed(const float p8[8], const PVIn &pv, WaveState &st)
{
    half2_t vpair[4][8];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) raw_pair<BITS>(pv.vc[2 * mm], pv.vc[2 * mm + 1], vpair[mm]);
    pv_mfma(p8, pv.sd, vpair, st);
}

// Stage A of a packed tile in LDS slot `slot`: Q K^T, softmax step, p -> pw (this wave's
// p buffer), and what stage B will need, copied out of the slot into registers. With MASK,
// tokens nvalid .. 31 of the tile are not attended (their logits are -inf). aq: the query
// octets divided by the key slots' weights, so the MFMA gives 2^-24 * sum_c q_c code_c;
// qs24: 2^-24 * sum(q over group g); sm24: 2^24 * sm_scale * log2(e).
template <int BITS, bool MASK = false>
__device__ __forceinline__ void stage_a_packed(const uint8_t *slot, float *pw, const half8_t aq[4],
                                               const float qs24[4], float sm24, int n, int r,
                                               WaveState &st, PVIn &pv, float &alpha,
                                               bool &rescale, int nvalid = kTile)
{
    using G = TileGeom<BITS>;
    const int gA = n & 3;
    KGroup<BITS> kc[2];
    u32x4 ksz[2], vsz[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        kc[u].load(slot, 16 * u + n, r);
        ksz[u] = *reinterpret_cast<const u32x4 *>(slot + G::KSZ + (16 * u + n) * 16);
        vsz[u] = *reinterpret_cast<const u32x4 *>(slot + G::VSZ + (16 * u + n) * 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pv.vc[e] = v_octet<BITS>(slot + G::CB, 4 * e + r, n);
        pv.sd[e] = *reinterpret_cast<const uint32_t *>(slot + G::VSZ + (4 * e + r) * 16 + 4 * gA);
    }

    float lg[2], zv[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < 4; ++o)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[o], kc[u].raw(o), acc, 0, 0, 0);
        // 2^-24 l = sum_g scale_g * dot_g + zero_g * sum(q over g), two chains of two groups
        float s01 = 0.0f, s23 = 0.0f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const half2_t a = as_h2(ksz[u][g]), c = as_h2(ksz[u][g + 2]);
            s01 = __builtin_fmaf((float)a.x, acc[g], s01);
            s01 = __builtin_fmaf((float)a.y, qs24[g], s01);
            s23 = __builtin_fmaf((float)c.x, acc[g + 2], s23);
            s23 = __builtin_fmaf((float)c.y, qs24[g + 2], s23);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) zv[u][g] = (float)as_h2(vsz[u][g]).y;
        lg[u] = (s01 + s23) * sm24;
        if (MASK && 16 * u + n >= nvalid) lg[u] = -INFINITY;
    }
    // any V scale of the tile at or above 2^(15 - kSlack)? (fp16 compare on the low halves)
    bool big = false;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) big |= as_h2(vsz[u][g]).x >= (_Float16)kBigScale;
    const bool big_scale = __builtin_amdgcn_ballot_w64(big) != 0;
    float p0, p1;
    softmax_a(lg, zv, big_scale, st, p0, p1, alpha, rescale);
    pw[p_pos(r, n)] = p0;
    pw[p_pos(r, 16 + n)] = p1;
}

__device__ __forceinline__ void rescale_pv(WaveState &st, float alpha)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) st.dpv[c] *= alpha;
}

// ---------------------------------------------------------------------------------------
// Outer-dimension groups (the KIVI-style comparison; a 32-token tile is exactly one token
// group, and the tile's scale/zero region holds {scale, zero} per channel). With per-
// channel scales the scale sits inside the Q K^T contraction, so it goes into the A
// operand: A = q * scale_k per channel, split into an fp16 high part and the fp16 of the
// remainder (two MFMAs, ~22 bits), B = the codes + 64 as before, and
//     l_t = sum_c (q s)_c (code + 64) + sum_c q_c (zero_c - 64 s_c).
// On the V side the scale varies along the output channels: each tile's P V (A = p, hi and
// lo) is taken into fresh accumulators and added as scale_c * (P V)_c + zero'_c * sum_t p_t.
// All of this is per tile, not per token.
// ---------------------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void stage_a_outer(const uint8_t *slot, float *pw, const uint16_t *qw,
                                              int NH, float sm_log2, const Magic &M, int n,
                                              int r, WaveState &st, PVInO &pv,
                                              float &alpha, bool &rescale)
{
    using G = TileGeom<BITS>;
    const int hA = n >> 2, gA = n & 3;
    const bool live = (gA == r) && (hA < NH);
    KGroup<BITS> kc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) kc[u].load(slot, 16 * u + n, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) pv.vc[e] = v_octet<BITS>(slot + G::CB, 4 * e + r, n);
    {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(slot + G::VSZ + 32 * n);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(slot + G::VSZ + 32 * n + 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pv.sz[k] = a[k];
            pv.sz[4 + k] = b[k];
        }
    }
    // octet o of the A operands (q * scale_k, hi and lo: channels 32 r + 8 o + i) is built
    // just before its four MFMAs (two tokens halves x hi/lo); this lane's part of
    // sum_c q_c zero'_c is summed on the way
    float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float zp = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        const int c0 = 32 * r + 8 * o;
        const u32x4 qv = *reinterpret_cast<const u32x4 *>(qw + 8 * q_piece(hA, r, o));
        const u32x4 s0 = *reinterpret_cast<const u32x4 *>(slot + G::KSZ + c0 * 4);
        const u32x4 s1 = *reinterpret_cast<const u32x4 *>(slot + G::KSZ + c0 * 4 + 16);
        u32x4 hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const half2_t q2 = as_h2(qv[k]);
            const uint32_t sa = k < 2 ? s0[2 * k] : s1[2 * k - 4];
            const uint32_t sb = k < 2 ? s0[2 * k + 1] : s1[2 * k - 3];
            const half2_t za = as_h2(sa), zb = as_h2(sb);      // {scale, zero} of the two channels
            const float qa = (float)q2.x, qb = (float)q2.y;
            const float pa = qa * (float)za.x, pb = qb * (float)zb.x;
            const _Float16 ha = (_Float16)pa, hb = (_Float16)pb;
            const _Float16 la = (_Float16)(pa - (float)ha), lb = (_Float16)(pb - (float)hb);
            hi[k] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
            lo[k] = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
            zp = __builtin_fmaf(qa, __builtin_fmaf(-64.0f, (float)za.x, (float)za.y), zp);
            zp = __builtin_fmaf(qb, __builtin_fmaf(-64.0f, (float)zb.x, (float)zb.y), zp);
        }
        const half8_t ah = live ? perm_octet_f16(hi) : half8_t{};
        const half8_t al = live ? perm_octet_f16(lo) : half8_t{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const half8_t kb = kc[u].octet(o, M);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, kb, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, kb, acc[u], 0, 0, 0);
        }
    }
    zp = live ? zp : 0.0f;
    // Z'_r = sum over the four groups of head r: lanes 16 g + 4 r + g hold them
    float zr = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
        zr += __int_as_float(__builtin_amdgcn_ds_bpermute((16 * g + 4 * r + g) * 4, __float_as_int(zp)));

    float lg[2], zv[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lg[u] = (((acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3])) + zr) * sm_log2;
#pragma unroll
        for (int g = 0; g < 4; ++g) zv[u][g] = 0.0f;
    }
    float p0, p1;
    softmax_a(lg, zv, false, st, p0, p1, alpha, rescale);
    pv.P = row_sum16(p0 + p1);
    pw[p_pos(r, n)] = p0;
    pw[p_pos(r, 16 + n)] = p1;
}

template <int BITS>
__device__ __forceinline__ void stage_b_outer(const float p8[8], const PVInO &pv, const Magic &M,
                                              WaveState &st)
{
    half2_t vpair[4][8];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) pair_tokens<BITS>(pv.vc[2 * mm], pv.vc[2 * mm + 1], M, vpair[mm]);
    u32x4 ahi, alo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ahi[k] = pv_hi(p8[2 * k], 0x3C00u, p8[2 * k + 1], 0x3C00u);
        alo[k] = pv_lo(p8[2 * k], 0x3C00u, p8[2 * k + 1], 0x3C00u, ahi[k]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const half8_t bv{vpair[0][c].x, vpair[0][c].y, vpair[1][c].x, vpair[1][c].y,
                         vpair[2][c].x, vpair[2][c].y, vpair[3][c].x, vpair[3][c].y};
        float4_t t = {0.f, 0.f, 0.f, 0.f};
        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ahi), bv, t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, alo), bv, t, 0, 0, 0);
        const half2_t sz = as_h2(pv.sz[c]);
        const float sc = (float)sz.x;
        const float zt = __builtin_fmaf(-64.0f, sc, (float)sz.y) * pv.P;   // zero' * sum p
        st.dpv[c] += sc * t + zt;
    }
}

// Merge the W waves' states of one workgroup through LDS (sm.mo, sm.ml). Thread t ends up
// with head h = t / 64 of the chunk and channels d, d + 1 (d = 2 * (t % 64)): the workgroup's
// normalised output o and its log-sum-exp in the exp2 domain (-inf, with o = 0, when the
// workgroup attended no token). Every wave of the workgroup must call it.
template <int NH, int W, class SM>
__device__ __forceinline__ void merge_waves(SM &sm, const WaveState &st, int wave, int n, int r,
                                            float &v0, float &v1, float &lse2)
{
    const float lsum = row_sum16(st.l);
    float zr[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) zr[g] = row_sum16(st.zacc[g]);
    {
        const int gj = n >> 2;   // group of channels 8n .. 8n+7
        const float zg = sel4(float4_t{zr[0], zr[1], zr[2], zr[3]}, gj);
        float4_t o0, o1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0[c] = sel4(st.dpv[c], gj) + zg;
            o1[c] = sel4(st.dpv[4 + c], gj) + zg;
        }
        float *mo = sm.mo(wave) + r * kHeadDim;
        *reinterpret_cast<float4_t *>(mo + 8 * n) = o0;
        *reinterpret_cast<float4_t *>(mo + 8 * n + 4) = o1;
        if (n == 0) {
            sm.ml[wave][r][0] = st.m;
            sm.ml[wave][r][1] = lsum;
        }
    }
    __syncthreads();
    const int h = threadIdx.x >> 6;       // 4 heads x 64 threads x 2 channels
    const int d = 2 * lane_full();
    v0 = 0.f;
    v1 = 0.f;
    lse2 = -INFINITY;
    if (h < NH) {
        // every wave's (m, l) and output pair read at once (one LDS round trip)
        float mw[W], lw[W];
        float2 ow[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            mw[w] = sm.ml[w][h][0];
            lw[w] = sm.ml[w][h][1];
            ow[w] = *reinterpret_cast<const float2 *>(sm.mo(w) + h * kHeadDim + d);
        }
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) Mx = fmaxf(Mx, mw[w]);
        // no branch (so the loads above are not moved behind one): with no attended token
        // in the workgroup every e is exp2(-inf) = 0 and L, o0, o1 stay 0
        const float Mref = Mx == -INFINITY ? 0.0f : Mx;
        float o0 = 0.f, o1 = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float e = __builtin_amdgcn_exp2f(mw[w] - Mref);
            L += e * lw[w];
            o0 += e * ow[w].x;
            o1 += e * ow[w].y;
        }
        if (L > 0.f) {
            const float inv = 1.0f / L;
            v0 = o0 * inv;
            v1 = o1 * inv;
            lse2 = Mx + __log2f(L);
        }
    }
}

// The split's partials: part_o (normalised) and part_lse (natural log) of the chunk's NH
// heads, query head hq0 + h.
template <int NH, int W, class SM>
__device__ __forceinline__ void merge_store(SM &sm, const WaveState &st, int wave, int n, int r,
                                            float *part_o, float *part_lse, int64_t hq0, int S,
                                            int split)
{
    float v0, v1, lse2;
    merge_waves<NH, W>(sm, st, wave, n, r, v0, v1, lse2);
    const int h = threadIdx.x >> 6;
    const int d = 2 * lane_full();
    if (h < NH) {
        const int64_t hq = hq0 + h;
        const int64_t ob = (hq * S + split) * kHeadDim + d;
        part_o[ob] = v0;
        part_o[ob + 1] = v1;
        if (d == 0) part_lse[hq * S + split] = lse2 == -INFINITY ? -INFINITY : lse2 * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------------------------------
// Split merge inside the decode launch (kvq_decode_attention_fused). The splits of one group
// (a row's head chunk) form a tree of fan-in 32 (one level up to 32 splits): every workgroup
// stores its record (the output of the chunk's heads and their log-sum-exp), then counts
// itself in its parent's counter; the last of a parent's (up to 32) children merges their
// records into the parent's record and goes up one level, and the last one at the top
// writes the output. Nobody waits
// for anybody, so the launch drains however its workgroups are scheduled.
// Records and counters are read and written with device-scope coherent accesses (the sc1
// cache policy: the L2 of each XCD passes them through), and a workgroup counts itself only
// after its record stores have completed (s_waitcnt vmcnt(0)), so the merging workgroup,
// which issues its loads after its counter update returned, sees every child's record
// wherever the children ran.
// Workspace: slots of kRecFloats words, kvq::fused_records(S) per group (a row's head
// chunk); for S = 1 none (the workgroup writes the output directly). A slot holds a record
// (4 heads x 128 outputs, then the 4 log2-domain log-sum-exps) and, in word kCtrWord, the
// counter of the parent whose first child the record is. Records never write that word and
// the workgroup that completes a parent puts its counter back to zero, so every counter
// word is zero again when a launch ends, whatever the shapes of the launches that share
// the workspace: the slot grid is the same for all of them.
constexpr int kRecFloats = 520;
constexpr int kCtrWord = 516;
constexpr int kScDevice = 16;            // sc1: device-scope coherent load / store

// Records are written and read by the workgroup's first 256 threads (4 heads x 64 threads x
// 2 channels); the threads of an eight-wave workgroup beyond them only join the barriers.
__device__ __forceinline__ void rec_store(__amdgpu_buffer_rsrc_t rr, int rec, float v0, float v1,
                                          float lse2)
{
    if (threadIdx.x >= 256) return;
    const int h = threadIdx.x >> 6;
    const int d = 2 * lane_full();
    const u32x2 v = {__float_as_uint(v0), __float_as_uint(v1)};
    __builtin_amdgcn_raw_buffer_store_b64(v, rr, (uint32_t)((rec * kRecFloats + h * kHeadDim + d) * 4),
                                          0, kScDevice);
    if (d == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2), rr,
                                              (uint32_t)((rec * kRecFloats + 4 * kHeadDim + h) * 4), 0,
                                              kScDevice);
}

// merge records first .. first + cnt - 1 (cnt <= kFanIn) into (v0, v1, lse2); all of a
// thread's loads are issued before the first is used (one memory round trip)
__device__ __forceinline__ void rec_merge(__amdgpu_buffer_rsrc_t rr, int first, int cnt, float &v0,
                                          float &v1, float &lse2)
{
    v0 = 0.f;
    v1 = 0.f;
    lse2 = -INFINITY;
    if (threadIdx.x >= 256) return;
    const int h = threadIdx.x >> 6;
    const int d = 2 * lane_full();
    u32x2 x[kFanIn];
    uint32_t lb[kFanIn];
#pragma unroll
    for (int j = 0; j < kFanIn; ++j) {
        // (cnt is uniform: a node with fewer children issues only their loads)
        if (j < cnt) {
            const int rec = first + j;
            x[j] = __builtin_amdgcn_raw_buffer_load_b64(rr, (uint32_t)((rec * kRecFloats + h * kHeadDim + d) * 4),
                                                        0, kScDevice);
            lb[j] = __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)((rec * kRecFloats + 4 * kHeadDim + h) * 4),
                                                         0, kScDevice);
        } else {
            x[j] = u32x2{0u, 0u};
            lb[j] = 0xff800000u;     // -inf: weighs nothing
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFanIn; ++j)
        if (j < cnt) M = fmaxf(M, __uint_as_float(lb[j]));
    float a0 = 0.f, a1 = 0.f, ws = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int j = 0; j < kFanIn; ++j) {
            if (j < cnt) {
                const float w = __builtin_amdgcn_exp2f(__uint_as_float(lb[j]) - M);
                a0 += w * __uint_as_float(x[j][0]);
                a1 += w * __uint_as_float(x[j][1]);
                ws += w;
            }
        }
    }
    if (ws > 0.f) {
        const float inv = 1.0f / ws;
        v0 = a0 * inv;
        v1 = a1 * inv;
        lse2 = M + __log2f(ws);
    } else {
        v0 = 0.f;
        v1 = 0.f;
        lse2 = -INFINITY;
    }
}

template <int NH>
__device__ __forceinline__ void out_store(const DecArgs &a, int64_t hq0, float v0, float v1)
{
    const int h = threadIdx.x >> 6;
    const int d = 2 * lane_full();
    if (h >= NH) return;
    const int64_t o = (hq0 + h) * kHeadDim + d;
    if (a.out_f16) {
        const half2_t hv = {(_Float16)v0, (_Float16)v1};
        *reinterpret_cast<half2_t *>(static_cast<uint16_t *>(a.out) + o) = hv;
    } else {
        *reinterpret_cast<float2 *>(static_cast<float *>(a.out) + o) = float2{v0, v1};
    }
}

template <int NH, int W, class SM>
__device__ __forceinline__ void merge_fused(SM &sm, const WaveState &st, int wave, int n, int r,
                                            const DecArgs &a, int64_t group, int64_t hq0, int split)
{
    float v0, v1, lse2;
    merge_waves<NH, W>(sm, st, wave, n, r, v0, v1, lse2);
    if (a.S == 1) {
        out_store<NH>(a, hq0, v0, v1);
        return;
    }
    float *recs = static_cast<float *>(a.ws) + group * a.rec_per_group * kRecFloats;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        recs, 0, a.rec_per_group * kRecFloats * 4, kRsrcWord3);
    int n_lvl = a.S, idx = split, rec0 = 0;
    rec_store(rr, idx, v0, v1, lse2);
    for (;;) {
        const int parent = idx / kFanIn, first = parent * kFanIn;
        const int cnt = n_lvl - first < kFanIn ? n_lvl - first : kFanIn;
        const int n_up = (n_lvl + kFanIn - 1) / kFanIn;
        if (cnt > 1) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this record is stored
            __syncthreads();
            if (threadIdx.x == 0) {
                uint32_t *c = reinterpret_cast<uint32_t *>(recs + (int64_t)(rec0 + first) * kRecFloats) +
                              kCtrWord;
                const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t last = old == (uint32_t)(cnt - 1);
                if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sm.flag = last;
            }
            __syncthreads();
            if (!sm.flag) return;
            rec_merge(rr, rec0 + first, cnt, v0, v1, lse2);
        }
        if (n_up == 1) {
            out_store<NH>(a, hq0, v0, v1);
            return;
        }
        rec0 += n_lvl;
        idx = parent;
        n_lvl = n_up;
        rec_store(rr, rec0 + idx, v0, v1, lse2);
    }
}

// Waves per SIMD that the LDS lets a CU hold (160 KB per CU, one Smem per workgroup of W
// waves), at most three. The inner-grouped kernels ask the register allocator for that
// occupancy (three waves per SIMD means at most 168 VGPRs); the outer-grouped comparison
// kernel needs more registers and asks for one.
template <int BITS, int RING, int W>
constexpr int lds_waves_per_simd()
{
    constexpr int wgs = (160 * 1024) / (int)sizeof(Smem<TileGeom<BITS>::BYTES, RING, W, 1>);
    constexpr int waves = wgs * W / 4;
    return waves < 1 ? 1 : (waves > 3 ? 3 : waves);
}

template <int BITS, int NH, int RING, int W, bool PAGED, bool OUTER = false, bool FUSED = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OUTER ? 1 : lds_waves_per_simd<BITS, RING, W>()))) void decode_kernel(DecArgs a,
                                                        const int32_t *__restrict__ tbl,
                                                        const int32_t *__restrict__ seq_state)
{
    using G = TileGeom<BITS>;
    static_assert(RING >= 2 && RING <= 8, "ring depth");
    static_assert(RING * G::BYTES >= 4 * kHeadDim * 4, "merge output must fit in a wave's ring");
    constexpr int kWaves = W;
    __shared__ Smem<G::BYTES, RING, W, 1> sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    const int n = lane & 15;
    const int r = lane >> 4;
    const int64_t row = blockIdx.x;                 // b * Hkv + kvh
    const int split = blockIdx.y;
    const int b = (int)(row / a.Hkv);
    const int kvh = (int)(row % a.Hkv);
    const int h0 = kvh * a.gq + a.head_base + blockIdx.z * 4;   // first query head of the chunk

    // ---- this sequence's lengths (a paged cache has its own per sequence) ----
    int n_packed_b = a.n_packed, n_res_b = a.n_res;
    int upd_slot = -1;      // update calls: the window slot the new token takes
    int ev_pos = -1;        // update calls that evict: the packed position of the evicted token
    if constexpr (PAGED) {
        n_packed_b = __builtin_amdgcn_readfirstlane(seq_state[4 * (int64_t)b]);
        n_res_b = __builtin_amdgcn_readfirstlane(seq_state[4 * (int64_t)b + 1]);
        if (a.upd) {
            // the step's update, as kvq_append_evict applies it (same clamping of a state
            // outside its range): the new token takes slot n_res while the window has room;
            // otherwise the token in slot next_slot moves to packed position n_packed and
            // the new token takes its slot. Attention then covers the updated lengths.
            const int nxt = __builtin_amdgcn_readfirstlane(seq_state[4 * (int64_t)b + 2]);
            const bool full = n_res_b >= a.res_cap;
            int slot = full ? nxt : (n_res_b < 0 ? 0 : n_res_b);
            if (full && (slot < a.n_sink || slot >= a.res_cap)) slot = a.n_sink;
            upd_slot = slot;
            const int n_packed_new = full ? n_packed_b + 1 : n_packed_b;
            const int n_res_new = full ? a.res_cap : slot + 1;
            if (full) ev_pos = n_packed_b;
            if (kvh == 0 && split == 0 && blockIdx.z == 0 && a.head_base == 0 && threadIdx.x == 0) {
                const int pad = seq_state[4 * (int64_t)b + 3];
                const int nxt_new = full ? (slot + 1 < a.res_cap ? slot + 1 : a.n_sink) : nxt;
                *reinterpret_cast<int4 *>(a.state_out + 4 * (int64_t)b) =
                    int4{n_packed_new, n_res_new, nxt_new, pad};
            }
            n_packed_b = n_packed_new;
            n_res_b = n_res_new;
        }
        // out-of-range lengths are clamped (never an access outside the table or window)
        const int cap_p = a.max_blocks * kBlockTokens;
        n_packed_b = n_packed_b < 0 ? 0 : (n_packed_b > cap_p ? cap_p : n_packed_b);
        n_res_b = n_res_b < 0 ? 0 : (n_res_b > a.res_cap ? a.res_cap : n_res_b);
    }

    // ---- token range of this split (same rule as the header documents) ----
    int tlo, thi;
    bool with_res;
    if constexpr (PAGED)
        split_range_seq(a, split, n_packed_b, n_res_b, tlo, thi, with_res);
    else
        split_range(a, split, tlo, thi, with_res);

    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.kp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.vp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);
    // the last tile of a ragged sequence: tokens nv_last .. 31 are past the sequence's end
    // (the pool bytes behind them may be anything). Their scale/zero words are loaded as
    // zeros (the block's buffer range ends at the last valid token's scale/zero word, and a
    // direct-to-LDS load past the range writes zeros), so their K and V dequantize to 0;
    // they are also masked out of the softmax.
    const int nt_seq = (n_packed_b + kTile - 1) / kTile;
    const int nv_last = n_packed_b - (nt_seq - 1) * kTile;
    // request tile `tile` of this row into `slot`: from the contiguous row, or from the
    // pool block the table names (a block id outside the pool reads block 0 instead)
    auto issue = [&](uint8_t *slot, int tile) {
        if constexpr (PAGED) {
            int64_t blk = __builtin_amdgcn_readfirstlane(tbl[(int64_t)b * a.max_blocks + (tile >> 2)]);
            if (blk < 0 || blk >= a.pool_blocks) blk = 0;
            const int64_t off = blk * a.block_stride + (int64_t)kvh * a.head_stride;
            const int tb0 = (tile & 3) * kTile;
            const int nrec = tile == nt_seq - 1 && nv_last < kTile
                                 ? a.sz_off + (tb0 + nv_last) * 16 : a.block_bytes;
            const __amdgpu_buffer_rsrc_t rkt = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(a.kp + off), 0, nrec, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rvt = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(a.vp + off), 0, nrec, kRsrcWord3);
            issue_tile_at<BITS>(rkt, rvt, slot, 0u, tb0, lane, a.sz_off);
        } else {
            issue_tile<BITS>(rk, rv, slot, tile, lane, a.block_bytes, a.sz_off);
        }
    };
    // An update that evicts: the wave that takes the tile holding the evicted token's new
    // packed position quantizes that token (the old contents of the window slot, staged in
    // sm.ev) exactly as kvq_append_evict does, writes it into its tile in LDS over whatever
    // the pool held there, stores it into the pool, and only then writes the new token into
    // the window slot. No other workgroup of the launch reads those pool bytes, and readers
    // of the slot take the new token from k_new / v_new.
    const int ev_tile = ev_pos >> 5;
    const bool ev_mine = PAGED && ev_pos >= 0 && ev_pos < n_packed_b && ev_tile >= tlo &&
                         ev_tile < thi && (ev_tile - tlo) % kWaves == wave;
    bool ev_mapped = false;
    // quantize the staged token (lanes 0..15 K, 16..31 V, one octet each), keep its bytes for
    // the tile in sm.evc / sm.evs, store it into the pool, then write the new token into the
    // window slot (run once, once the staging load is in)
    auto evict_token = [&]() {
        if constexpr (PAGED) {
            const int oct = lane & 15;
            const int is_v = (lane >> 4) & 1;
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(&sm.ev[is_v][8 * oct]);
            uint32_t packed;
            uint16_t sq, zq;
            int flag;
            if (a.hybrid) quantize_octet<BITS, true>(raw, packed, sq, zq, flag);
            else quantize_octet<BITS, false>(raw, packed, sq, zq, flag);
            PoolGeom g{const_cast<uint8_t *>(is_v ? a.vp : a.kp), a.pool_blocks, a.block_stride,
                       a.head_stride, tbl, a.max_blocks, a.sz_off, a.flag_off};
            uint8_t *blk = block_of(g, b, kvh, ev_pos);
            if (lane < 32) {
                sm.evc[is_v][oct] = packed;
                if ((oct & 3) == 0) sm.evs[is_v][oct >> 2] = (uint32_t)sq | ((uint32_t)zq << 16);
                if (blk) {
                    if (a.hybrid) store_octet<BITS, true>(blk, g, ev_pos & 127, oct, packed, sq, zq, flag);
                    else store_octet<BITS, false>(blk, g, ev_pos & 127, oct, packed, sq, zq, flag);
                }
                uint16_t *win = const_cast<uint16_t *>(is_v ? a.vres : a.kres) +
                                (row * a.res_cap + upd_slot) * kHeadDim + 8 * oct;
                *reinterpret_cast<u32x4 *>(win) =
                    *reinterpret_cast<const u32x4 *>(&sm.ev[2 + is_v][8 * oct]);
            }
            ev_mapped = blk != nullptr;
            lds_fence();
        }
    };
    // the kept bytes into token ev_pos % 32 of the tile in LDS (over whatever the pool held)
    auto evict_patch = [&](uint8_t *slot) {
        const int t = ev_pos & 31;
        const int oct = lane & 15;
        const int is_v = (lane >> 4) & 1;
        if (lane < 32 && ev_mapped) {
            const uint32_t packed = sm.evc[is_v][oct];
            const int grp = oct >> 2, jq = oct & 3;
            uint8_t *cb = slot + (is_v ? G::CB : 0);
            if (!is_v && BITS == 4) {
                // the transposed order of 4-bit K codes in LDS (issue_tile_at)
                *reinterpret_cast<uint32_t *>(cb + (t >> 4) * 1024 + grp * 256 + (t & 15) * 16 +
                                              jq * 4) = packed;
            } else if (!is_v && BITS == 2) {
                // the transposed order of 2-bit K codes in LDS (issue_tile_at)
                *reinterpret_cast<uint16_t *>(cb + (t >> 4) * 512 + (grp >> 1) * 256 + (t & 15) * 16 +
                                              (grp & 1) * 8 + jq * 2) = (uint16_t)packed;
            } else {
                uint8_t *c = cb + t * G::TOKB + grp * (4 * BITS) + jq * BITS;
                if (BITS == 4) {
                    *reinterpret_cast<uint32_t *>(c) = packed;
                } else if (BITS == 2) {
                    *reinterpret_cast<uint16_t *>(c) = (uint16_t)packed;
                } else {
                    c[0] = (uint8_t)packed;
                    c[1] = (uint8_t)(packed >> 8);
                    c[2] = (uint8_t)(packed >> 16);
                }
            }
            if (jq == 0)
                *reinterpret_cast<uint32_t *>(slot + (is_v ? G::VSZ : G::KSZ) + t * 16 + grp * 4) =
                    sm.evs[is_v][grp];
        }
    };
    // the number of valid tokens of a tile once it is in LDS; the tile of an update's
    // evicted token (the sequence's last packed token, so its last tile) is patched first
    auto tail_fix = [&](uint8_t *slot, int tile) -> int {
        if constexpr (PAGED) {
            if (tile == nt_seq - 1) {
                if (ev_mine) {
                    evict_patch(slot);
                    lds_fence();
                }
                return nv_last;
            }
        }
        return kTile;
    };

    // ---- q of the chunk's heads -> this wave's LDS copy (one 1 KB direct-to-LDS load,
    // issued before the tile requests so it is the oldest outstanding load) ----
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q), 0, a.q_bytes, kRsrcWord3);
    // (wave 0 stages q for the whole workgroup, and the row's 128 key-channel norms when q
    // is to be multiplied by them; both straight into LDS, so that no load into registers is
    // in flight next to the tile loads: the compiler would wait for all loads before
    // reusing such a register)
    if (wave == 0) {
        dma(rq, reinterpret_cast<uint8_t *>(&sm.q[0][0][0]),
            (uint32_t)(((int64_t)b * a.Hq + h0) * kHeadDim * 2) + q_piece_src(lane) * 16, 16);
        if (a.qnorm && lane < 32) {
            const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float *>(a.qnorm + row * kHeadDim), 0, kHeadDim * 4, kRsrcWord3);
            dma(rn, reinterpret_cast<uint8_t *>(&sm.qn[0]), lane * 16, 16);
        }
    }

    // the evicted token's old window contents and the new token, staged before this wave's
    // tiles are asked for: they are older than every tile load waited for, so no wait of
    // their own (a plain load here would have to wait for every load in flight)
    if (ev_mine && lane < 16) {
        const int64_t wrow = (row * a.res_cap + upd_slot) * kHeadDim;
        const __amdgpu_buffer_rsrc_t rek = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.kres + wrow), 0, kHeadDim * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rev = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vres + wrow), 0, kHeadDim * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rnk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.knew + row * kHeadDim), 0, kHeadDim * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rnv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.vnew + row * kHeadDim), 0, kHeadDim * 2, kRsrcWord3);
        dma(rek, reinterpret_cast<uint8_t *>(&sm.ev[0][0]), lane * 16, 16);
        dma(rev, reinterpret_cast<uint8_t *>(&sm.ev[1][0]), lane * 16, 16);
        dma(rnk, reinterpret_cast<uint8_t *>(&sm.ev[2][0]), lane * 16, 16);
        dma(rnv, reinterpret_cast<uint8_t *>(&sm.ev[3][0]), lane * 16, 16);
    }

    // ---- ask for this wave's first RING tiles ----
    const int my_lo = tlo + wave;
    const int nt_w = my_lo < thi ? (thi - my_lo + kWaves - 1) / kWaves : 0;
    uint8_t *ring = &sm.ring[wave][0][0];
    // Only the first tile is asked for before the prologue (q, A operands), the rest right
    // after it: the first tiles of all waves then reach the memory system ahead of the
    // second ones (measured 0.2 us faster at 32K tokens than asking for both at once).
    constexpr int kFirst = 1;
#pragma unroll
    for (int k = 0; k < kFirst; ++k)
        if (k < nt_w) issue(ring + k * G::BYTES, my_lo + k * kWaves);
    if (wave == 0) wait_behind<BITS>(nt_w < kFirst ? nt_w : kFirst);   // q, issued before the tiles
    if (wave == 0 && a.qnorm) {
        // q' = fp16(q * norm) per channel: lane (r, n) rescales the 16 bytes it loaded
        // (head r of the chunk, channels 8n..8n+7) in place
        u32x4 *mine = reinterpret_cast<u32x4 *>(&sm.q[0][0][0]) + q_piece(r, n >> 2, n & 3);
        const u32x4 w = *mine;
        const float4_t qn0 = *reinterpret_cast<const float4_t *>(&sm.qn[8 * n]);
        const float4_t qn1 = *reinterpret_cast<const float4_t *>(&sm.qn[8 * n + 4]);
        const float nv[8] = {qn0[0], qn0[1], qn0[2], qn0[3], qn1[0], qn1[1], qn1[2], qn1[3]};
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const half2_t h = as_h2(w[k]);
            float y0 = (float)h.x * nv[2 * k], y1 = (float)h.y * nv[2 * k + 1];
            asm("" : "+v"(y0), "+v"(y1));     // binary32 product, then its own fp16 rounding
            o[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
        }
        *mine = o;
    }
    // q in LDS for every wave. A plain s_barrier: __syncthreads would also wait for this
    // wave's tile loads (the compiler counts direct-to-LDS loads as LDS writes to release),
    // while only wave 0's q (waited for above) and its q' stores must be complete here.
    lds_fence();
    __builtin_amdgcn_s_barrier();

    // ---- QK A operands and per-group sums sum_{c in g} q_h[c] ----
    // The query octets in the key operand's slot order; for the packed tiles slot pair p is
    // divided by the weight 2^raw_key_shift(p) its subnormal codes carry (exact in fp16 but
    // for values that become subnormal; the fp16 window rebuilds them undivided).
    half8_t aq[4];
    auto build_aq = [&](bool weighted) {
        const int hA = n >> 2, gA = n & 3;
        const bool live = (gA == r) && (hA < NH);
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const u32x4 w = reinterpret_cast<const u32x4 *>(&sm.q[0][0][0])[q_piece(hA, r, o)];
            half8_t h = live ? perm_octet_f16(w) : half8_t{};
            if (weighted) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    h[i] = (_Float16)((float)h[i] * (1.0f / (float)(1 << raw_key_shift<BITS>(i >> 1))));
            }
            aq[o] = h;
        }
    };
    build_aq(!OUTER);
#pragma unroll
    for (int k = kFirst; k < RING; ++k)
        if (k < nt_w) issue(ring + k * G::BYTES, my_lo + k * kWaves);
    float qs[4];
    {
        // lane (hh, gg, qq) sums 8 channels; the quad sum is Qs[hh][gg]; lane (n, r) then
        // fetches Qs[r][g] from lane 16r + 4g
        const int hh = lane >> 4, gg = (lane >> 2) & 3, qq = lane & 3;
        const u32x4 v = reinterpret_cast<const u32x4 *>(&sm.q[0][0][0])[q_piece(hh, gg, qq)];
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const half2_t hv = as_h2(v[k]);
            s += (float)hv.x + (float)hv.y;
        }
        s = hh < NH ? s : 0.0f;
        s += dpp_f<0xB1>(s);
        s += dpp_f<0x4E>(s);
#pragma unroll
        for (int g = 0; g < 4; ++g)
            qs[g] = __int_as_float(__builtin_amdgcn_ds_bpermute((16 * r + 4 * g) * 4, __float_as_int(s)));
    }
    const float qs24[4] = {qs[0] * 0x1p-24f, qs[1] * 0x1p-24f, qs[2] * 0x1p-24f, qs[3] * 0x1p-24f};
    const float sm24 = a.sm_log2 * 0x1p24f;

    const Magic M;
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.zacc[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.dpv[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    using PV = std::conditional_t<OUTER, PVInO, PVIn>;
    const uint16_t *qw = &sm.q[0][0][0];
    // stage A / stage B of one packed tile, for the inner or the outer grouping
    auto stage_a = [&](const uint8_t *slot, float *pw, PV &pv, float &alpha, bool &resc, int nv) {
        if constexpr (OUTER) {
            (void)nv;
            stage_a_outer<BITS>(slot, pw, qw, NH, a.sm_log2, M, n, r, st, pv, alpha, resc);
        } else {
            stage_a_packed<BITS, PAGED>(slot, pw, aq, qs24, sm24, n, r, st, pv, alpha, resc, nv);
        }
    };
    auto stage_b = [&](const float p8[8], const PV &pv) {
        if constexpr (OUTER) stage_b_outer<BITS>(p8, pv, M, st);
        else stage_b_packed<BITS>(p8, pv, st);
    };

    // ---- packed tiles through the ring, software-pipelined ----
    // Iteration k runs stage B (P V) of tile k next to stage A (Q K^T, softmax, p) of
    // tile k+1, so one wave has two independent chains of work. RING tiles are requested up
    // front; once stage A of tile j has read its slot, tile j + RING is requested into it,
    // so RING - 1 tiles stay in flight behind the one being read.
    float *pbuf = &sm.p[wave][0][0][0];
    const int pstride = 4 * kTile;
    if (nt_w > 0) {
        wait_behind<BITS>(nt_w - 1 < RING - 1 ? nt_w - 1 : RING - 1);
        if (ev_mine) evict_token();      // its staging load is older than the tile just waited for
        PV cur;
        float alpha;
        bool resc;
        const int nv0 = tail_fix(ring, my_lo);
        stage_a(ring, pbuf, cur, alpha, resc, nv0);
        wait_lgkm0();                                    // slot 0 read, p of tile 0 written
        if (RING < nt_w) issue(ring, my_lo + RING * kWaves);
        // one pipeline step: stage A of tile k+1 (into `nxt`) next to stage B of tile k
        auto step = [&](int k, const PV &cur, PV &nxt) {
            // tile k+1 in LDS; the tiles up to k+RING may still be in flight
            wait_behind<BITS>(nt_w - 2 - k < RING - 1 ? nt_w - 2 - k : RING - 1);
            set_prio(nt_w - k);
            const int s1 = (k + 1) % RING;
            const int nv = tail_fix(ring + s1 * G::BYTES, my_lo + (k + 1) * kWaves);
            float p8[8];
            load_p8(pbuf + (k & 1) * pstride, n, r, p8);
            if constexpr (OUTER) {
                stage_a(ring + s1 * G::BYTES, pbuf + ((k + 1) & 1) * pstride, nxt, alpha, resc, nv);
                stage_b(p8, cur);
            } else {
                // P V of tile k first: its operands are ready at the top of the step, so
                // its MFMAs overlap the unpack and softmax of tile k+1, and fewer values
                // stay live across the step (the same arithmetic in either order)
                stage_b(p8, cur);
                stage_a(ring + s1 * G::BYTES, pbuf + ((k + 1) & 1) * pstride, nxt, alpha, resc, nv);
            }
            if (resc) rescale_pv(st, alpha);      // tile k's PV is in; tile k+1 moved m
            wait_lgkm0();                                // slot k+1 read, p of tile k+1 written
            if (k + 1 + RING < nt_w) issue(ring + s1 * G::BYTES, my_lo + (k + 1 + RING) * kWaves);
        };
        auto last = [&](int k, const PV &cur) {
            float p8[8];
            load_p8(pbuf + (k & 1) * pstride, n, r, p8);
            stage_b(p8, cur);
            wait_lgkm0();
        };
        // two steps per trip so that the stage-A output and stage-B input swap roles
        // instead of being copied
        PV nxt;
        int k = 0;
        for (; k + 2 < nt_w; k += 2) {
            step(k, cur, nxt);
            step(k + 1, nxt, cur);
        }
        if (k + 1 < nt_w) {
            step(k, cur, nxt);
            last(k + 1, nxt);
        } else {
            last(k, cur);
        }
        if constexpr (!OUTER) {
            // the V codes entered as subnormals: column c of every octet weighed
            // 2^(raw_value_shift(c) - 24); back to value units (exact)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                st.dpv[c] *= (float)(1 << (24 - raw_value_shift<BITS>(c)));
        }
    }

    // ---- residual / sink tokens (fp16), in 32-token tiles ----
    if (with_res) {
        if constexpr (!OUTER) build_aq(false);
        const uint16_t *kr = a.kres + row * a.res_cap * kHeadDim;
        const uint16_t *vr = a.vres + row * a.res_cap * kHeadDim;
        // a new token (kvq_decode_attention_append) is window slot n_res - 1: it is read
        // from k_new / v_new here, and the workgroup of the row's first query heads (first
        // chunk of the launch that starts at head 0) stores it into the window; every
        // reader of that slot in these launches reads k_new / v_new instead
        // (a paged update places the new token at upd_slot; when it evicts, the slot is
        // written by the wave that moves the old token out, after reading it)
        const int new_slot = (PAGED && a.upd) ? upd_slot : (a.knew ? n_res_b - 1 : -1);
        const uint16_t *kn = a.knew ? a.knew + row * kHeadDim : kr;
        const uint16_t *vn = a.vnew ? a.vnew + row * kHeadDim : vr;
        if (new_slot >= 0 && ev_pos < 0 && a.head_base == 0 && blockIdx.z == 0 && threadIdx.x < 32) {
            const bool is_v = threadIdx.x >= 16;
            const int t = threadIdx.x & 15;
            uint16_t *dst = const_cast<uint16_t *>(is_v ? vr : kr) + (int64_t)new_slot * kHeadDim + 8 * t;
            *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>((is_v ? vn : kn) + 8 * t);
        }
        const int n_rt = (n_res_b + kTile - 1) / kTile;
        for (int rt = wave; rt < n_rt; rt += kWaves) {
            float lg[2], zv[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ts = rt * kTile + 16 * u + n;
                const int tc = ts < n_res_b ? ts : n_res_b - 1;
                const uint16_t *kt = (tc == new_slot ? kn : kr + (int64_t)tc * kHeadDim) + 32 * r;
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int o = 0; o < 4; ++o)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        aq[o], perm_octet_f16(*reinterpret_cast<const u32x4 *>(kt + 8 * o)), acc, 0, 0, 0);
                const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                lg[u] = ts < n_res_b ? s * a.sm_log2 : -INFINITY;
#pragma unroll
                for (int g = 0; g < 4; ++g) zv[u][g] = 0.0f;
            }
            u32x4 vt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ts = rt * kTile + 4 * e + r;
                const int tc = ts < n_res_b ? ts : n_res_b - 1;
                vt[e] = *reinterpret_cast<const u32x4 *>((tc == new_slot ? vn : vr + (int64_t)tc * kHeadDim) + 8 * n);
            }
            half2_t vpair[4][8];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    vpair[mm][c] = as_h2((c & 1) ? pack_hi16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1])
                                                 : pack_lo16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1]));
            float p0, p1, alpha;
            bool resc;
            softmax_a(lg, zv, false, st, p0, p1, alpha, resc);
            if (resc) rescale_pv(st, alpha);
            pbuf[p_pos(r, n)] = p0;
            pbuf[p_pos(r, 16 + n)] = p1;
            lds_fence();
            float p8[8];
            load_p8(pbuf, n, r, p8);
            uint32_t ones[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ones[e] = 0x3C00u;   // fp16 1.0: window tokens are not scaled
            pv_mfma(p8, ones, vpair, st);
            lds_fence();                                     // p read before the next tile rewrites it
        }
    }

    // ---- merge the waves; write this split's partials, or merge the splits here ----
    if constexpr (FUSED)
        merge_fused<NH, W>(sm, st, wave, n, r, a, row * a.n_chunks + (a.head_base >> 2) + blockIdx.z,
                           (int64_t)b * a.Hq + h0, split);
    else
        merge_store<NH, W>(sm, st, wave, n, r, a.part_o, a.part_lse, (int64_t)b * a.Hq + h0, a.S,
                           split);
}

// ---------------------------------------------------------------------------------------
// FP16 flash-decoding baseline: the same split-K partials from an uncompressed fp16 K/V
// cache (rows of [tokens][128], token-major), the decode the packed cache is compared
// against (BitDecoding page sec. 4.2 reports its speed-ups over FP16 decoding). Same
// workgroup layout, ring of direct-to-LDS loads, MFMA Q K^T / P V and merge as the packed
// kernel, with fp16 K and V operands in place of the codes.
// ---------------------------------------------------------------------------------------
constexpr int kF16TokB = kHeadDim * 2;                 // 256 B per token
constexpr int kF16TileB = 2 * kTile * kF16TokB;        // K rows, then V rows: 16 KB
constexpr int kF16NI = kF16TileB / 1024;               // 16 direct-to-LDS loads per tile

__device__ __forceinline__ void issue_tile_f16(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                               uint8_t *slot, int tile, int lane)
{
    const uint32_t base = (uint32_t)tile * (kTile * kF16TokB);
#pragma unroll
    for (int k = 0; k < kTile * kF16TokB / 1024; ++k) {
        dma_nt(rk, slot + 1024 * k, base + 1024 * k + lane * 16);
        dma_nt(rv, slot + kTile * kF16TokB + 1024 * k, base + 1024 * k + lane * 16);
    }
}

// wait until the oldest outstanding load group is in LDS with `after` (0..2) younger fp16
// tiles still in flight behind it
__device__ __forceinline__ void wait_behind_f16(int after)
{
    if (after >= 2) wait_vm<2 * kF16NI>();
    else if (after == 1) wait_vm<kF16NI>();
    else wait_vm<0>();
}

template <int NH, int W>
__global__ __launch_bounds__(64 * W) void decode_f16_kernel(DecArgs a)
{
    constexpr int kWaves = W;
    __shared__ Smem<kF16TileB, 2, W> sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int r = lane >> 4;
    const int64_t row = blockIdx.x;
    const int split = blockIdx.y;
    const int b = (int)(row / a.Hkv);
    const int kvh = (int)(row % a.Hkv);
    const int h0 = kvh * a.gq + a.head_base + blockIdx.z * 4;

    const int L = a.n_res;                             // tokens in the fp16 cache
    const int NT = (L + kTile - 1) / kTile;
    const int tlo = (int)((int64_t)split * NT / a.S);
    const int thi = (int)((int64_t)(split + 1) * NT / a.S);

    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.kres + row * a.row_stride * kHeadDim), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.vres + row * a.row_stride * kHeadDim), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q), 0, a.q_bytes, kRsrcWord3);
    dma(rq, reinterpret_cast<uint8_t *>(&sm.q[wave][0][0]),
        (uint32_t)(((int64_t)b * a.Hq + h0) * kHeadDim * 2) + lane * 16, 16);

    const int my_lo = tlo + wave;
    const int nt_w = my_lo < thi ? (thi - my_lo + kWaves - 1) / kWaves : 0;
    uint8_t *ring = &sm.ring[wave][0][0];
#pragma unroll
    for (int k = 0; k < 2; ++k)
        if (k < nt_w) issue_tile_f16(rk, rv, ring + k * kF16TileB, my_lo + k * kWaves, lane);
    wait_behind_f16(nt_w < 2 ? nt_w : 2);              // q, issued before the tiles

    half8_t aq[4];
    {
        const int hA = n >> 2, gA = n & 3;
        const bool live = (gA == r) && (hA < NH);
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.q[wave][hA][32 * r + 8 * o]);
            aq[o] = live ? perm_octet_f16(w) : half8_t{};
        }
    }
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.zacc[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.dpv[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    float *pbuf = &sm.p[wave][0][0][0];
    uint32_t ones[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = 0x3C00u;     // fp16 1.0: fp16 tokens are not scaled

    for (int k = 0; k < nt_w; ++k) {
        wait_behind_f16(k + 1 < nt_w ? 1 : 0);
        set_prio(nt_w - k);
        const uint8_t *slot = ring + (k & 1) * kF16TileB;
        const int tok0 = (my_lo + k * kWaves) * kTile;
        float lg[2], zv[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 16 * u + n;
            const uint8_t *kt = slot + t * kF16TokB + r * 64;
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int o = 0; o < 4; ++o)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    aq[o], perm_octet_f16(*reinterpret_cast<const u32x4 *>(kt + 16 * o)), acc, 0, 0, 0);
            const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            lg[u] = tok0 + t < L ? s * a.sm_log2 : -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; ++g) zv[u][g] = 0.0f;
        }
        u32x4 vt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vt[e] = *reinterpret_cast<const u32x4 *>(slot + kTile * kF16TokB + (4 * e + r) * kF16TokB + 16 * n);
        half2_t vpair[4][8];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                vpair[mm][c] = as_h2((c & 1) ? pack_hi16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1])
                                             : pack_lo16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1]));
        float p0, p1, alpha;
        bool resc;
        softmax_a(lg, zv, false, st, p0, p1, alpha, resc);
        if (resc) rescale_pv(st, alpha);
        pbuf[p_pos(r, n)] = p0;
        pbuf[p_pos(r, 16 + n)] = p1;
        lds_fence();
        float p8[8];
        load_p8(pbuf, n, r, p8);
        pv_mfma(p8, ones, vpair, st);
        wait_lgkm0();                                  // slot and p read
        if (k + 2 < nt_w) issue_tile_f16(rk, rv, ring + (k & 1) * kF16TileB, my_lo + (k + 2) * kWaves, lane);
    }
    merge_store<NH, W>(sm, st, wave, n, r, a.part_o, a.part_lse, (int64_t)b * a.Hq + h0, a.S, split);
}

template <int NH>
hipError_t launch_f16_nh(const DecArgs &a, int64_t rows, int chunks, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_f16_kernel<NH, 4>), dim3((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

#ifndef KVQ_RING
#define KVQ_RING 2
#endif
// Ring depth per wave: two slots (three workgroups per CU). Deeper rings, which keep more
// tiles in flight per wave but leave fewer waves per CU, measured slower at every grid
// size tried (e.g. 16.6 us with 7 slots and one workgroup per CU against 12.4 us with
// 2 slots at 32K tokens), because the first tiles arrive later and one wave per SIMD
// computes its tiles more slowly.

template <int BITS, int NH, int R, int W, bool PAGED = false, bool FUSED = false>
hipError_t launch_r(const DecArgs &a, dim3 grid, hipStream_t stream, const int32_t *tbl = nullptr)
{
    hipLaunchKernelGGL((decode_kernel<BITS, NH, R, W, PAGED, false, FUSED>), grid, dim3(64 * W), 0,
                       stream, a, tbl, a.state);
    return hipGetLastError();
}

// Compute units of the current device (looked up once per device).
int cu_count()
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cus[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Workgroup shape: when the grid has no more workgroups than the device has compute units,
// each gets a CU of its own and eight waves (two per SIMD) share the split's tiles; with
// more workgroups, four-wave workgroups let two or three of them share a CU.
template <int BITS, bool PAGED, bool FUSED>
hipError_t launch_bits(const DecArgs &a, const int32_t *tbl, int nh, int64_t rows, int chunks,
                       int64_t total_wgs, hipStream_t stream)
{
    const dim3 grid((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks);
#ifndef KVQ_WIDE
#define KVQ_WIDE 8
#endif
    if (total_wgs <= cu_count()) {
        switch (nh) {
        case 1: return launch_r<BITS, 1, KVQ_RING, KVQ_WIDE, PAGED, FUSED>(a, grid, stream, tbl);
        case 2: return launch_r<BITS, 2, KVQ_RING, KVQ_WIDE, PAGED, FUSED>(a, grid, stream, tbl);
        case 3: return launch_r<BITS, 3, KVQ_RING, KVQ_WIDE, PAGED, FUSED>(a, grid, stream, tbl);
        case 4: return launch_r<BITS, 4, KVQ_RING, KVQ_WIDE, PAGED, FUSED>(a, grid, stream, tbl);
        default: return hipErrorInvalidValue;
        }
    }
    switch (nh) {
    case 1: return launch_r<BITS, 1, KVQ_RING, 4, PAGED, FUSED>(a, grid, stream, tbl);
    case 2: return launch_r<BITS, 2, KVQ_RING, 4, PAGED, FUSED>(a, grid, stream, tbl);
    case 3: return launch_r<BITS, 3, KVQ_RING, 4, PAGED, FUSED>(a, grid, stream, tbl);
    case 4: return launch_r<BITS, 4, KVQ_RING, 4, PAGED, FUSED>(a, grid, stream, tbl);
    default: return hipErrorInvalidValue;
    }
}

template <bool PAGED, bool FUSED>
hipError_t launch_nh(const DecArgs &a, const int32_t *tbl, int bits, int nh, int64_t rows,
                     int chunks, int64_t total_wgs, hipStream_t stream)
{
    switch (bits) {
    case 2: return launch_bits<2, PAGED, FUSED>(a, tbl, nh, rows, chunks, total_wgs, stream);
    case 3: return launch_bits<3, PAGED, FUSED>(a, tbl, nh, rows, chunks, total_wgs, stream);
    case 4: return launch_bits<4, PAGED, FUSED>(a, tbl, nh, rows, chunks, total_wgs, stream);
    default: return hipErrorInvalidValue;
    }
}

// the launches of one decode call: the full 4-head chunks of every row, then (gq % 4 != 0)
// one launch for the remaining heads of every row
template <bool PAGED, bool FUSED>
hipError_t launch_chunks(DecArgs a, const int32_t *tbl, int bits, int64_t rows, hipStream_t stream)
{
    const int full = a.gq / 4, tail = a.gq % 4;
    const int64_t total_wgs = rows * a.S * (full + (tail > 0));
    hipError_t e = hipSuccess;
    if (full > 0) {
        a.head_base = 0;
        e = launch_nh<PAGED, FUSED>(a, tbl, bits, 4, rows, full, total_wgs, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) {
        a.head_base = full * 4;
        e = launch_nh<PAGED, FUSED>(a, tbl, bits, tail, rows, 1, total_wgs, stream);
    }
    return e;
}

// outer-grouped blocks: the default ring depth only
template <int BITS>
hipError_t launch_outer_bits(const DecArgs &a, int nh, int64_t rows, int chunks,
                             hipStream_t stream)
{
    constexpr int W = 4;
    const dim3 grid((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks);
    switch (nh) {
    case 1: hipLaunchKernelGGL((decode_kernel<BITS, 1, KVQ_RING, W, false, true>), grid, dim3(64 * W), 0, stream, a, nullptr, nullptr); break;
    case 2: hipLaunchKernelGGL((decode_kernel<BITS, 2, KVQ_RING, W, false, true>), grid, dim3(64 * W), 0, stream, a, nullptr, nullptr); break;
    case 3: hipLaunchKernelGGL((decode_kernel<BITS, 3, KVQ_RING, W, false, true>), grid, dim3(64 * W), 0, stream, a, nullptr, nullptr); break;
    case 4: hipLaunchKernelGGL((decode_kernel<BITS, 4, KVQ_RING, W, false, true>), grid, dim3(64 * W), 0, stream, a, nullptr, nullptr); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_outer_nh(const DecArgs &a, int bits, int nh, int64_t rows, int chunks,
                           hipStream_t stream)
{
    switch (bits) {
    case 2: return launch_outer_bits<2>(a, nh, rows, chunks, stream);
    case 3: return launch_outer_bits<3>(a, nh, rows, chunks, stream);
    case 4: return launch_outer_bits<4>(a, nh, rows, chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_f16_heads(const DecArgs &a, int nh, int64_t rows, int chunks, hipStream_t stream)
{
    switch (nh) {
    case 1: return launch_f16_nh<1>(a, rows, chunks, stream);
    case 2: return launch_f16_nh<2>(a, rows, chunks, stream);
    case 3: return launch_f16_nh<3>(a, rows, chunks, stream);
    case 4: return launch_f16_nh<4>(a, rows, chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_f16(const DecodeParams &p, hipStream_t stream)
{
    DecArgs a = make_dec_args(p);
    a.row_stride = p.res_cap;                          // tokens between rows
    a.row_bytes = (int32_t)((int64_t)p.n_res * kF16TokB);
    const int64_t rows = (int64_t)p.B * p.Hkv;
    const int full = a.gq / 4, tail = a.gq % 4;
    hipError_t e = hipSuccess;
    if (full > 0) {
        a.head_base = 0;
        e = launch_f16_heads(a, 4, rows, full, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) {
        a.head_base = full * 4;
        e = launch_f16_heads(a, tail, rows, 1, stream);
    }
    return e;
}

static DecArgs paged_args(const DecodeParams &p)
{
    DecArgs a = make_dec_args(p);
    a.row_stride = 0;
    a.row_bytes = 0;
    a.n_packed = 0;     // per sequence, from the state
    a.n_res = 0;
    return a;
}

hipError_t launch_decode_paged(const DecodeParams &p, hipStream_t stream)
{
    return launch_chunks<true, false>(paged_args(p), p.tbl, p.bits, (int64_t)p.B * p.Hkv, stream);
}

hipError_t launch_decode_paged_fused(const DecodeParams &p, hipStream_t stream)
{
    return launch_chunks<true, true>(paged_args(p), p.tbl, p.bits, (int64_t)p.B * p.Hkv, stream);
}

hipError_t launch_decode_outer(const DecodeParams &p, hipStream_t stream)
{
    DecArgs a = make_dec_args(p);
    const int64_t rows = (int64_t)p.B * p.Hkv;
    const int full = a.gq / 4, tail = a.gq % 4;
    hipError_t e = hipSuccess;
    if (full > 0) {
        a.head_base = 0;
        e = launch_outer_nh(a, p.bits, 4, rows, full, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) {
        a.head_base = full * 4;
        e = launch_outer_nh(a, p.bits, tail, rows, 1, stream);
    }
    return e;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream)
{
    return launch_chunks<false, false>(make_dec_args(p), nullptr, p.bits, (int64_t)p.B * p.Hkv,
                                       stream);
}

hipError_t launch_decode_fused(const DecodeParams &p, hipStream_t stream)
{
    return launch_chunks<false, true>(make_dec_args(p), nullptr, p.bits, (int64_t)p.B * p.Hkv,
                                      stream);
}


// ---------------------------------------------------------------------------------------
// Scratch of the allocation-free fused decode (kvq_decode_attention_fused_noalloc): the
// split records and counters live in this array instead of a caller workspace. Every GPU
// the library runs on holds its own copy until the process ends, and every call on that
// GPU shares it. In host code `scratch` only stands in for the symbol: the kernels get the
// device address that hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint8_t *p, size_t n)
{
    const size_t n16 = n / 16;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        reinterpret_cast<u32x4 *>(p)[i] = u32x4{0u, 0u, 0u, 0u};
}

// the array's address on the current device: looked up, and zeroed by a kernel on
// `stream`, at the first call on that device
hipError_t scratch_on_device(void **ptr, hipStream_t stream)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(512), dim3(256), 0, stream,
                           static_cast<uint8_t *>(p), kScratchBytes);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode_fused_noalloc(DecodeParams p, hipStream_t stream)
{
    if (fused_workspace_bytes(p.B, p.Hq, p.Hkv, p.num_splits) > (int64_t)kScratchBytes)
        return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = scratch_on_device(&ws, stream);
    if (e != hipSuccess) return e;
    p.ws = ws;
    return launch_decode_fused(p, stream);
}

}  // namespace kvq
