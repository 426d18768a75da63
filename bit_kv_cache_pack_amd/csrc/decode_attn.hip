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
//    2-slot ring per wave: a wave asks for its next two tiles up front and for tile k+2
//    as soon as tile k is consumed, so ~10 KB per wave (120 KB per CU at three resident
//    workgroups) is in flight without holding it in VGPRs; the wave waits on vmcnt for
//    exactly the tile it is about to use.
//  * Q K^T uses v_mfma_f32_16x16x32_f16 with B = the raw integer codes (exact in fp16,
//    made with the fp16 magic-number trick) and rows i = 4*head + group of A holding the
//    query restricted to one 32-channel group. Lane (token n, r) loads group r of token n
//    (one 16/12/8-byte load), and MFMA o consumes that group's channel octet o, so the
//    result row 4h+g is head h's dot product with group g's codes. Every lane then holds
//    the four group dots of one (token, head) and applies its token's scale/zero:
//        l = sum_g scale_g * dot_g + zero_g * sum(q over g)
//    with no cross-lane reduction.
//  * P V uses the same MFMA with rows i = 4*head + group holding p * scale_v (split into
//    an fp16 high part and an fp16 remainder, two MFMAs, so the weights keep ~22 bits)
//    and B = the V codes of 8 tokens x 1 channel per lane, built from two tokens' code
//    words at a time. Only rows whose group matches the column's group are used; the
//    zero-point term sum_t p_t zero_v is accumulated on the VALU.
//  * row (16-lane) max / sum reductions use DPP; p and scale_v pass through a 1 KB
//    per-wave LDS slice to reach the PV operand layout.
#include "kvq_device.h"
#include "kvq_internal.h"

#include <math.h>

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;
// a tile's max may exceed the running max by up to 2^kSlack before the accumulators are
// rescaled; p * scale_v then stays below 65504 whenever scale_v < 2^(15 - kSlack)
constexpr float kSlack = 8.0f;
constexpr float kBigScale = 128.0f;   // 2^(15 - kSlack)
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer access, gfx9 family

struct DecArgs {
    const uint16_t *q;
    int32_t q_bytes;             // bytes of q, the range its buffer resource covers
    int32_t Hq, Hkv, gq, head_base;
    const uint8_t *kp, *vp;
    int64_t row_stride;
    int32_t row_bytes;           // bytes of a packed row the kernel may touch
    int32_t n_packed;
    const uint16_t *kres, *vres;
    int32_t res_cap, n_res;
    float sm_log2;               // sm_scale * log2(e): logits are kept in the exp2 domain
    int32_t S, Sp, res_alone;
    float *part_o, *part_lse;
    int32_t block_bytes, sz_off;
};

constexpr int kRing = 2;

// LDS of one workgroup, ~48 KB at 4 bits, so that three workgroups (12 waves) share a CU.
// A wave's merge output (mo) reuses the start of its own ring once its tiles are done.
template <int TILE_BYTES>
struct Smem {
    alignas(16) uint8_t ring[kWaves][kRing][TILE_BYTES];   // per-wave ring of staged tiles
    alignas(16) uint16_t q[kWaves][4][kHeadDim];            // per-wave copy of the chunk's q
    alignas(16) float p[kWaves][4][kTile];    // p of head h, token t of the current tile
    alignas(16) float sv[kWaves][4][kTile];   // V scale of group g, token t
    alignas(16) float ml[kWaves][4][2];
    __device__ __forceinline__ float *mo(int w) { return reinterpret_cast<float *>(&ring[w][0][0]); }
};
static_assert(kRing * 1024 * 3 >= 4 * kHeadDim * 4, "merge output must fit in a wave's ring");

__device__ __forceinline__ void lds_fence()
{
    // finish this wave's LDS traffic before its lanes read what other lanes wrote
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// 8 fp16 values (natural channel order, 16 bytes) -> slot order (0,4,1,5,2,6,3,7)
__device__ __forceinline__ half8_t perm_octet_f16(u32x4 w)
{
    const half2_t a = as_h2(pack_lo16(w[0], w[2]));
    const half2_t b = as_h2(pack_hi16(w[0], w[2]));
    const half2_t c = as_h2(pack_lo16(w[1], w[3]));
    const half2_t d = as_h2(pack_hi16(w[1], w[3]));
    return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

typedef __attribute__((address_space(3))) void lds_void;

// Tile geometry in LDS: K codes | V codes | K scale/zero | V scale/zero, each in the
// order the packed block stores them (32 tokens).
template <int BITS>
struct TileGeom {
    static constexpr int TOKB = kHeadDim * BITS / 8;   // code bytes per token
    static constexpr int GB = 4 * BITS;                // code bytes per group
    static constexpr int CB = kTile * TOKB;            // code bytes per tile (2048/1536/1024)
    static constexpr int KSZ = 2 * CB;                 // offset of K scale/zero (512 B)
    static constexpr int VSZ = 2 * CB + 512;           // offset of V scale/zero (512 B)
    static constexpr int BYTES = 2 * CB + 1024;
    static constexpr int NI = (BITS == 2 ? 2 : 4) + 2; // direct-to-LDS loads per tile
};
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint8_t *lds, uint32_t voff, int size)
{
    // 16 bytes per lane; lane i's bytes land at lds + 16 * i (lds is wave-uniform)
    (void)size;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, 0, 0, 0);
}

// Ask for packed tile `tile` (32 tokens) of this row: K and V codes and scale/zero.
template <int BITS>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           uint8_t *slot, int tile, int lane, int block_bytes,
                                           int sz_off)
{
    using G = TileGeom<BITS>;
    const int tok0 = tile * kTile;
    const uint32_t blk = (uint32_t)(tok0 >> 7) * (uint32_t)block_bytes;
    const int tb0 = tok0 & 127;
    const uint32_t c0 = blk + tb0 * G::TOKB;
    if (BITS == 3) {          // 1536 B = 64 lanes x 16 B + 32 lanes x 16 B
        dma(rk, slot, c0 + lane * 16, 16);
        dma(rv, slot + G::CB, c0 + lane * 16, 16);
        if (lane < 32) {
            dma(rk, slot + 1024, c0 + 1024 + lane * 16, 16);
            dma(rv, slot + G::CB + 1024, c0 + 1024 + lane * 16, 16);
        }
    } else {
#pragma unroll
        for (int k = 0; k < G::CB / 1024; ++k) {
            dma(rk, slot + 1024 * k, c0 + 1024 * k + lane * 16, 16);
            dma(rv, slot + G::CB + 1024 * k, c0 + 1024 * k + lane * 16, 16);
        }
    }
    if (lane < 32) {          // 32 tokens x 16 B of scale/zero each for K and V
        const uint32_t s0 = blk + sz_off + tb0 * 16 + lane * 16;
        dma(rk, slot + G::KSZ, s0, 16);
        dma(rv, slot + G::VSZ, s0, 16);
    }
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// wait until tile k is in LDS, when `after` (< kRing) younger tiles may still be in flight
template <int BITS>
__device__ __forceinline__ void wait_tile(int after)
{
    constexpr int NI = TileGeom<BITS>::NI;
    static_assert(kRing == 2, "one younger tile at most");
    if (after >= 1) wait_vm<NI>();
    else wait_vm<0>();
}

// wait for the q copy, requested before `tiles` (0..kRing) tiles
template <int BITS>
__device__ __forceinline__ void wait_q(int tiles)
{
    constexpr int NI = TileGeom<BITS>::NI;
    if (tiles >= 2) wait_vm<2 * NI>();
    else if (tiles == 1) wait_vm<NI>();
    else wait_vm<0>();
}

// K codes of token t (0..31 in the tile), group r, as channel octets
template <int BITS>
struct KGroup;
template <>
struct KGroup<4> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint8_t *slot, int t, int r)
    {
        w = *reinterpret_cast<const u32x4 *>(slot + t * 64 + r * 16);
    }
    __device__ __forceinline__ half8_t octet(int o, const Magic &M) const { return unpack_octet4(w[o], M); }
};
template <>
struct KGroup<2> {
    u32x2 w;
    __device__ __forceinline__ void load(const uint8_t *slot, int t, int r)
    {
        w = *reinterpret_cast<const u32x2 *>(slot + t * 32 + r * 8);
    }
    __device__ __forceinline__ half8_t octet(int o, const Magic &M) const
    {
        return unpack_octet2((o & 1) ? (w[o >> 1] >> 16) : w[o >> 1], M);
    }
};
template <>
struct KGroup<3> {
    uint32_t w0, w1, w2;
    __device__ __forceinline__ void load(const uint8_t *slot, int t, int r)
    {
        const uint32_t *d = reinterpret_cast<const uint32_t *>(slot + t * 48 + r * 12);
        w0 = d[0];
        w1 = d[1];
        w2 = d[2];
    }
    __device__ __forceinline__ half8_t octet(int o, const Magic &M) const
    {
        const uint32_t x = o == 0 ? w0 : o == 1 ? __builtin_amdgcn_alignbit(w1, w0, 24)
                                     : o == 2 ? __builtin_amdgcn_alignbit(w2, w1, 16) : (w2 >> 8);
        return unpack_octet3(x, M);
    }
};

// V codes of channel octet j of token t of the tile (low bits of the result)
template <int BITS>
__device__ __forceinline__ uint32_t v_octet(const uint8_t *vcodes, int t, int j)
{
    if (BITS == 4) return reinterpret_cast<const uint32_t *>(vcodes + t * 64)[j];
    if (BITS == 2) return reinterpret_cast<const uint16_t *>(vcodes + t * 32)[j];
    // 3 bits: bytes 3j..3j+2 of the 48-byte row, from the two dwords that cover them
    // (for t = 31, j = 15 the second dword is the first of the K scale/zero region, in
    // the same slot)
    const uint32_t byte = 3 * j;
    const uint32_t *d = reinterpret_cast<const uint32_t *>(vcodes + t * 48 + (byte & ~3u));
    return __builtin_amdgcn_alignbit(d[1], d[0], (byte & 3u) * 8);
}

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

// v[k] for a lane-varying k in 0..3, as two levels of selects (a runtime vector index
// would otherwise go through scratch memory)
__device__ __forceinline__ float sel4(float4_t v, int k)
{
    const float a = (k & 1) ? v[1] : v[0];
    const float b = (k & 1) ? v[3] : v[2];
    return (k & 2) ? b : a;
}
__device__ __forceinline__ uint32_t sel4u(u32x4 v, int k)
{
    const uint32_t a = (k & 1) ? v[1] : v[0];
    const uint32_t b = (k & 1) ? v[3] : v[2];
    return (k & 2) ? b : a;
}

// Online-softmax state of one wave: lane (n, r) tracks head r.
struct WaveState {
    float m, l;
    float zacc[4];     // sum_t p_t * zero'_v(t, g) for head r, group g (lane partial)
    float4_t dpv[8];   // PV accumulators: rows 4h+g, column n <-> channel 8n + c
};

// Softmax update and PV for one 32-token tile. lg[u]: logits (exp2 domain) of token
// 16u + n for head r; zv[u][g]: V zero-point term of that token; vpair[m][c]: the V
// operand pair (slots 2m, 2m+1 of lane group r, i.e. tokens 8m + r and 8m + 4 + r;
// channel 8n + c). The V scale of (token, group r) is already in sm.sv.
template <int NH, class SM>
__device__ __forceinline__ void softmax_pv(SM &sm, int wave, int n, int r, const float lg[2],
                                           const float zv[2][4], const half2_t vpair[4][8],
                                           bool big_scale, WaveState &st)
{
    // Lazy rescale: the reference max m only moves when the tile's max exceeds it by more
    // than 2^kSlack (log2 units), or exceeds it at all while a V scale is so large that
    // p * scale could leave the fp16 range of the PV operand; otherwise p <= 2^kSlack.
    const float tmax = row_max16(fmaxf(lg[0], lg[1]));
    const bool grow = (tmax > st.m + kSlack) || (big_scale && tmax > st.m);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float mnew = grow ? tmax : st.m;
        const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
        st.m = mnew;
        st.l *= alpha;
#pragma unroll
        for (int g = 0; g < 4; ++g) st.zacc[g] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.dpv[c] *= alpha;
    }
    const float p0 = __builtin_amdgcn_exp2f(lg[0] - st.m);
    const float p1 = __builtin_amdgcn_exp2f(lg[1] - st.m);
    st.l += p0 + p1;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.zacc[g] = __builtin_fmaf(p1, zv[1][g], __builtin_fmaf(p0, zv[0][g], st.zacc[g]));

    sm.p[wave][r][slot_pos(n)] = p0;
    sm.p[wave][r][slot_pos(16 + n)] = p1;
    lds_fence();

    // A operand of PV: lane (i, r) holds rows i = 4h + g, token slots 8r .. 8r+7
    const int hA = n >> 2, gA = n & 3;
    const float4_t pl = *reinterpret_cast<const float4_t *>(&sm.p[wave][hA][8 * r]);
    const float4_t ph = *reinterpret_cast<const float4_t *>(&sm.p[wave][hA][8 * r + 4]);
    const float4_t sl = *reinterpret_cast<const float4_t *>(&sm.sv[wave][gA][8 * r]);
    const float4_t sh = *reinterpret_cast<const float4_t *>(&sm.sv[wave][gA][8 * r + 4]);
    const float w[8] = {pl[0] * sl[0], pl[1] * sl[1], pl[2] * sl[2], pl[3] * sl[3],
                        ph[0] * sh[0], ph[1] * sh[1], ph[2] * sh[2], ph[3] * sh[3]};
    half8_t ahi, alo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = hA < NH ? w[e] : 0.0f;
        const _Float16 hi = (_Float16)x;
        ahi[e] = hi;
        alo[e] = (_Float16)(x - (float)hi);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const half8_t bv{vpair[0][c].x, vpair[0][c].y, vpair[1][c].x, vpair[1][c].y,
                         vpair[2][c].x, vpair[2][c].y, vpair[3][c].x, vpair[3][c].y};
        st.dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, st.dpv[c], 0, 0, 0);
        st.dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, st.dpv[c], 0, 0, 0);
    }
    // the next tile rewrites sm.p / sm.sv only after these reads have returned
    lds_fence();
}

template <int BITS, int NH, class SM>
__device__ __forceinline__ void packed_tile(SM &sm, const uint8_t *slot, const half8_t aq[4],
                                            const float qs[4], float sm_log2, const Magic &M,
                                            int wave, int n, int r, WaveState &st)
{
    using G = TileGeom<BITS>;
    KGroup<BITS> kc[2];
    u32x4 ksz[2], vsz[2];
    uint32_t vc[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        kc[u].load(slot, 16 * u + n, r);
        ksz[u] = *reinterpret_cast<const u32x4 *>(slot + G::KSZ + (16 * u + n) * 16);
        vsz[u] = *reinterpret_cast<const u32x4 *>(slot + G::VSZ + (16 * u + n) * 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vc[e] = v_octet<BITS>(slot + G::CB, 4 * e + r, n);

    float lg[2], zv[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < 4; ++o)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[o], kc[u].octet(o, M), acc, 0, 0, 0);
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const half2_t szk = as_h2(ksz[u][g]);
            s = __builtin_fmaf((float)szk.x, acc[g], s);
            s = __builtin_fmaf((float)szk.y, qs[g], s);
            const half2_t szv = as_h2(vsz[u][g]);
            // the V operand carries codes + 64: zero' = zero - 64 * scale
            zv[u][g] = __builtin_fmaf(-64.0f, (float)szv.x, (float)szv.y);
        }
        lg[u] = s * sm_log2;
        sm.sv[wave][r][slot_pos(16 * u + n)] = (float)as_h2(sel4u(vsz[u], r)).x;
    }
    // any V scale of the tile at or above 2^(15 - kSlack)? (fp16 compare on the low halves)
    bool big = false;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) big |= as_h2(vsz[u][g]).x >= (_Float16)kBigScale;
    const bool big_scale = __builtin_amdgcn_ballot_w64(big) != 0;
    half2_t vpair[4][8];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) pair_tokens<BITS>(vc[2 * mm], vc[2 * mm + 1], M, vpair[mm]);
    softmax_pv<NH>(sm, wave, n, r, lg, zv, vpair, big_scale, st);
}

template <int BITS, int NH>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a)
{
    using G = TileGeom<BITS>;
    __shared__ Smem<G::BYTES> sm;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int r = lane >> 4;
    const int64_t row = blockIdx.x;                 // b * Hkv + kvh
    const int split = blockIdx.y;
    const int b = (int)(row / a.Hkv);
    const int kvh = (int)(row % a.Hkv);
    const int h0 = kvh * a.gq + a.head_base + blockIdx.z * 4;   // first query head of the chunk

    // ---- token range of this split (same rule as the header documents) ----
    const int NT = a.n_packed / kTile;
    int tlo = 0, thi = 0;
    bool with_res;
    if (a.res_alone && split == a.S - 1) {
        with_res = true;
    } else {
        tlo = (int)((int64_t)split * NT / a.Sp);
        thi = (int)((int64_t)(split + 1) * NT / a.Sp);
        with_res = !a.res_alone && split == a.S - 1;
    }
    with_res = with_res && a.n_res > 0;

    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.kp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.vp + row * a.row_stride), 0, a.row_bytes, kRsrcWord3);

    // ---- q of the chunk's heads -> this wave's LDS copy (one 1 KB direct-to-LDS load,
    // issued before the tile requests so it is the oldest outstanding load) ----
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.q), 0, a.q_bytes, kRsrcWord3);
    dma(rq, reinterpret_cast<uint8_t *>(&sm.q[wave][0][0]),
        (uint32_t)(((int64_t)b * a.Hq + h0) * kHeadDim * 2) + lane * 16, 16);

    // ---- ask for this wave's first tiles ----
    const int my_lo = tlo + wave;
    const int nt_w = my_lo < thi ? (thi - my_lo + kWaves - 1) / kWaves : 0;
    uint8_t *ring = &sm.ring[wave][0][0];
#pragma unroll
    for (int k = 0; k < kRing; ++k)
        if (k < nt_w) issue_tile<BITS>(rk, rv, ring + k * G::BYTES, my_lo + k * kWaves, lane,
                                       a.block_bytes, a.sz_off);
    wait_q<BITS>(nt_w < kRing ? nt_w : kRing);

    // ---- QK A operands and per-group sums sum_{c in g} q_h[c] ----
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
    float qs[4];
    {
        // lane (hh, gg, qq) sums 8 channels; the quad sum is Qs[hh][gg]; lane (n, r) then
        // fetches Qs[r][g] from lane 16r + 4g
        const int hh = lane >> 4, gg = (lane >> 2) & 3, qq = lane & 3;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(&sm.q[wave][hh][gg * 32 + qq * 8]);
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

    const Magic M;
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.zacc[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.dpv[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    // ---- packed tiles through the ring ----
    for (int k = 0; k < nt_w; ++k) {
        const int left = nt_w - 1 - k;                  // younger tiles possibly in flight
        wait_tile<BITS>(left < kRing - 1 ? left : kRing - 1);
        uint8_t *slot = ring + (k % kRing) * G::BYTES;
        packed_tile<BITS, NH>(sm, slot, aq, qs, a.sm_log2, M, wave, n, r, st);
        wait_lgkm0();                                    // the slot has been read
        if (k + kRing < nt_w)
            issue_tile<BITS>(rk, rv, slot, my_lo + (k + kRing) * kWaves, lane, a.block_bytes, a.sz_off);
    }

    // ---- residual / sink tokens (fp16), in 32-token tiles ----
    if (with_res) {
        const uint16_t *kr = a.kres + row * a.res_cap * kHeadDim;
        const uint16_t *vr = a.vres + row * a.res_cap * kHeadDim;
        const int n_rt = (a.n_res + kTile - 1) / kTile;
        for (int rt = wave; rt < n_rt; rt += kWaves) {
            float lg[2], zv[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ts = rt * kTile + 16 * u + n;
                const int tc = ts < a.n_res ? ts : a.n_res - 1;
                const uint16_t *kt = kr + (int64_t)tc * kHeadDim + 32 * r;
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int o = 0; o < 4; ++o)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        aq[o], perm_octet_f16(*reinterpret_cast<const u32x4 *>(kt + 8 * o)), acc, 0, 0, 0);
                const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                lg[u] = ts < a.n_res ? s * a.sm_log2 : -INFINITY;
#pragma unroll
                for (int g = 0; g < 4; ++g) zv[u][g] = 0.0f;
                sm.sv[wave][r][slot_pos(16 * u + n)] = 1.0f;
            }
            u32x4 vt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ts = rt * kTile + 4 * e + r;
                const int tc = ts < a.n_res ? ts : a.n_res - 1;
                vt[e] = *reinterpret_cast<const u32x4 *>(vr + (int64_t)tc * kHeadDim + 8 * n);
            }
            half2_t vpair[4][8];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    vpair[mm][c] = as_h2((c & 1) ? pack_hi16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1])
                                                 : pack_lo16(vt[2 * mm][c >> 1], vt[2 * mm + 1][c >> 1]));
            softmax_pv<NH>(sm, wave, n, r, lg, zv, vpair, false, st);
        }
    }

    // ---- merge the waves ----
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
    {
        const int h = threadIdx.x >> 6;       // 4 heads x 64 threads x 2 channels
        const int d = (threadIdx.x & 63) * 2;
        if (h < NH) {
            float Mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, sm.ml[w][h][0]);
            float o0 = 0.f, o1 = 0.f, L = 0.f;
            if (Mx != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float e = __builtin_amdgcn_exp2f(sm.ml[w][h][0] - Mx);
                    L += e * sm.ml[w][h][1];
                    o0 += e * sm.mo(w)[h * kHeadDim + d];
                    o1 += e * sm.mo(w)[h * kHeadDim + d + 1];
                }
            }
            const int64_t hq = (int64_t)b * a.Hq + h0 + h;
            const int64_t ob = (hq * a.S + split) * kHeadDim + d;
            float v0 = 0.f, v1 = 0.f, lse = -INFINITY;
            if (L > 0.f) {
                const float inv = 1.0f / L;
                v0 = o0 * inv;
                v1 = o1 * inv;
                lse = (Mx + __log2f(L)) * 0.69314718055994531f;
            }
            a.part_o[ob] = v0;
            a.part_o[ob + 1] = v1;
            if (d == 0) a.part_lse[hq * a.S + split] = lse;
        }
    }
}

template <int BITS, int NH>
hipError_t launch_t(const DecArgs &a, int64_t rows, int chunks, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_kernel<BITS, NH>),
                       dim3((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const DecArgs &a, int nh, int64_t rows, int chunks, hipStream_t stream)
{
    switch (nh) {
    case 1: return launch_t<BITS, 1>(a, rows, chunks, stream);
    case 2: return launch_t<BITS, 2>(a, rows, chunks, stream);
    case 3: return launch_t<BITS, 3>(a, rows, chunks, stream);
    case 4: return launch_t<BITS, 4>(a, rows, chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nh(const DecArgs &a, int bits, int nh, int64_t rows, int chunks, hipStream_t stream)
{
    switch (bits) {
    case 2: return launch_bits<2>(a, nh, rows, chunks, stream);
    case 3: return launch_bits<3>(a, nh, rows, chunks, stream);
    case 4: return launch_bits<4>(a, nh, rows, chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream)
{
    DecArgs a{};
    a.q = p.q;
    a.q_bytes = (int32_t)((int64_t)p.B * p.Hq * kHeadDim * 2);
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.gq = p.Hq / p.Hkv;
    a.kp = p.kp;
    a.vp = p.vp;
    a.row_stride = p.row_stride;
    a.n_packed = p.n_packed;
    a.kres = p.kres;
    a.vres = p.vres;
    a.res_cap = p.res_cap;
    a.n_res = p.n_res;
    a.sm_log2 = p.sm_scale * 1.4426950408889634f;
    a.S = p.num_splits;
    a.res_alone = (p.num_splits > 1 && p.n_res > 0) ? 1 : 0;
    a.Sp = a.res_alone ? p.num_splits - 1 : p.num_splits;
    a.part_o = p.part_o;
    a.part_lse = p.part_lse;
    a.block_bytes = p.block_bytes;
    a.sz_off = p.sz_off;
    a.row_bytes = (int32_t)((int64_t)(p.n_packed / kBlockTokens) * p.block_bytes);
    const int64_t rows = (int64_t)p.B * p.Hkv;
    const int full = a.gq / 4, tail = a.gq % 4;
    hipError_t e = hipSuccess;
    if (full > 0) {
        a.head_base = 0;
        e = launch_nh(a, p.bits, 4, rows, full, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) {
        a.head_base = full * 4;
        e = launch_nh(a, p.bits, tail, rows, 1, stream);
    }
    return e;
}

}  // namespace kvq
