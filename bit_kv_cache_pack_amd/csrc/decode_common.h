// decode_common.h -- pieces shared by the two decode kernels (the MFMA kernel in
// decode_attn.hip and the VALU comparison kernel in decode_valu.hip): kernel arguments,
// the 32-token tile layout in LDS, the direct-to-LDS tile loads and their vmcnt waits,
// code access in a staged tile, and the fp16 split of P*V weights.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

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
    const float *qnorm;          // key-channel norms [rows][128] q is multiplied by, or null
    const uint16_t *knew, *vnew; // new token [rows][128] for window slot n_res - 1, or null
    // paged cache (kp / vp are then the pools): block e of sequence b at
    // pool + tbl[b][e] * block_stride + kvh * head_stride; lengths from state[b][0..1]
    int32_t max_blocks;
    int64_t pool_blocks, block_stride, head_stride;
    const int32_t *state;
    // the update folded into a paged decode (DecodeParams::upd): state is read, the new
    // state goes to state_out; hybrid / flag_off describe the blocks the evicted token
    // is written into
    int32_t upd, n_sink, hybrid, flag_off;
    int32_t *state_out;
    // split merge inside the launch: the output [B][Hq][128] (fp32, or fp16 when out_f16),
    // the workspace of record slots, the slots per group, and the number of head chunks per
    // row (groups are (row, chunk))
    void *out;
    int32_t out_f16;
    void *ws;
    int32_t rec_per_group, n_chunks;
};

// The lane index, counted from the exec mask (valid where all 64 lanes are active, as in
// the merge code after a workgroup barrier): a computation of its own, so the compiler does
// not keep threadIdx.x & 63 in a register from the start of the kernel to its end.
__device__ __forceinline__ int lane_full()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

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
// The same for cache data, which every launch reads exactly once: the non-temporal policy
// (nt) keeps the stream from displacing reusable lines in L2 and the Infinity Cache; it
// took a stream of the 4-bit tile layout at 32K tokens from 9.2 to 8.4 us per launch.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ void dma_nt(__amdgpu_buffer_rsrc_t r, uint8_t *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, 0, 0, kNonTemporal);
}

// Ask for the 32 tokens tb0 .. tb0+31 of the packed block at byte offset `blk` of the
// K and V buffer resources: their codes and scale/zero.
template <int BITS>
__device__ __forceinline__ void issue_tile_at(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                              uint8_t *slot, uint32_t blk, int tb0, int lane,
                                              int sz_off)
{
    using G = TileGeom<BITS>;
    const uint32_t c0 = blk + tb0 * G::TOKB;
    if (BITS == 3) {          // 1536 B = 64 lanes x 16 B + 32 lanes x 16 B
        dma_nt(rk, slot, c0 + lane * 16);
        dma_nt(rv, slot + G::CB, c0 + lane * 16);
        if (lane < 32) {
            dma_nt(rk, slot + 1024, c0 + 1024 + lane * 16);
            dma_nt(rv, slot + G::CB + 1024, c0 + 1024 + lane * 16);
        }
    } else {
        // K codes land with their 16-byte pieces transposed in LDS, so that the reads of
        // one group for 16 tokens hit every bank once (no conflict): at 4 bits each 1 KB
        // request (16 tokens x 64 B) puts the piece of group r of token n at position
        // 16 r + n (KGroup<4>::load); at 2 bits each 512 B half (16 tokens x 32 B) puts
        // piece j (groups 2j, 2j+1) of token n at position 16 j + n (KGroup<2>::load).
        // A request still reads the same whole 1 KB.
        const uint32_t koff = BITS == 4 ? (uint32_t)(64 * (lane & 15) + 16 * (lane >> 4))
                                        : (uint32_t)(512 * (lane >> 5) + 32 * (lane & 15) +
                                                     16 * ((lane >> 4) & 1));
#pragma unroll
        for (int k = 0; k < G::CB / 1024; ++k) {
            dma_nt(rk, slot + 1024 * k, c0 + 1024 * k + koff);
            dma_nt(rv, slot + G::CB + 1024 * k, c0 + 1024 * k + lane * 16);
        }
    }
    if (lane < 32) {          // 32 tokens x 16 B of scale/zero each for K and V
        const uint32_t s0 = blk + sz_off + tb0 * 16 + lane * 16;
        dma_nt(rk, slot + G::KSZ, s0);
        dma_nt(rv, slot + G::VSZ, s0);
    }
}

// Ask for packed tile `tile` (32 tokens) of a contiguous row.
template <int BITS>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           uint8_t *slot, int tile, int lane, int block_bytes,
                                           int sz_off)
{
    const int tok0 = tile * kTile;
    issue_tile_at<BITS>(rk, rv, slot, (uint32_t)(tok0 >> 7) * (uint32_t)block_bytes, tok0 & 127,
                        lane, sz_off);
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// wait until the oldest outstanding load group is in LDS, when `after` (0..7) younger
// tiles may still be in flight behind it
template <int BITS>
__device__ __forceinline__ void wait_behind(int after)
{
    constexpr int NI = TileGeom<BITS>::NI;
    static_assert(7 * NI < 64, "vmcnt range");
    switch (after < 7 ? after : 7) {
    case 7: wait_vm<7 * NI>(); break;
    case 6: wait_vm<6 * NI>(); break;
    case 5: wait_vm<5 * NI>(); break;
    case 4: wait_vm<4 * NI>(); break;
    case 3: wait_vm<3 * NI>(); break;
    case 2: wait_vm<2 * NI>(); break;
    case 1: wait_vm<NI>(); break;
    default: wait_vm<0>(); break;
    }
}

// Wave priority for instruction issue from the number of tiles the wave still has to
// process (more left -> higher): without it the older of two workgroups sharing a CU wins
// every issue conflict and the younger one finishes last.
__device__ __forceinline__ void set_prio(int left)
{
    if (left >= 4) __builtin_amdgcn_s_setprio(3);
    else if (left == 3) __builtin_amdgcn_s_setprio(2);
    else if (left == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// K codes of token t (0..31 in the tile), group r, as channel octets
template <int BITS>
struct KGroup;
template <>
struct KGroup<4> {
    u32x4 w;
    // group r of token t: piece 16 r + t % 16 of the tokens' 1 KB half (the transposed
    // order issue_tile_at writes)
    __device__ __forceinline__ void load(const uint8_t *slot, int t, int r)
    {
        w = *reinterpret_cast<const u32x4 *>(slot + (t >> 4) * 1024 + r * 256 + (t & 15) * 16);
    }
    __device__ __forceinline__ half8_t octet(int o, const Magic &M) const { return unpack_octet4(w[o], M); }
    __device__ __forceinline__ half8_t raw(int o) const { return raw_octet4(w[o]); }
};
template <>
struct KGroup<2> {
    u32x2 w;
    // group r of token t: half r % 2 of piece 16 (r / 2) + t % 16 of the tokens' 512 B half
    // (the transposed order issue_tile_at writes)
    __device__ __forceinline__ void load(const uint8_t *slot, int t, int r)
    {
        w = *reinterpret_cast<const u32x2 *>(slot + (t >> 4) * 512 + (r >> 1) * 256 + (t & 15) * 16 +
                                             (r & 1) * 8);
    }
    __device__ __forceinline__ half8_t octet(int o, const Magic &M) const
    {
        return unpack_octet2((o & 1) ? (w[o >> 1] >> 16) : w[o >> 1], M);
    }
    __device__ __forceinline__ half8_t raw(int o) const
    {
        return raw_octet2((o & 1) ? (w[o >> 1] >> 16) : w[o >> 1]);
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
    __device__ __forceinline__ half8_t raw(int o) const
    {
        const uint32_t x = o == 0 ? w0 : o == 1 ? __builtin_amdgcn_alignbit(w1, w0, 24)
                                     : o == 2 ? __builtin_amdgcn_alignbit(w2, w1, 16) : (w2 >> 8);
        return raw_octet3(x);
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

// fp16 pair {hi(p0 * s0), hi(p1 * s1)}: each product of the fp32 p and the fp16 scale
// (the low half of a {scale, zero} dword) formed in fp32 and rounded to fp16; the compiler
// emits one v_fma_mix per half. (Written in C, not inline asm, so that the compiler sees
// these VALU writes and keeps the wait states the MFMA that reads them needs.)
__device__ __forceinline__ uint32_t pv_hi(float p0, uint32_t s0, float p1, uint32_t s1)
{
    const _Float16 a = (_Float16)__builtin_fmaf(p0, (float)as_h2(s0)[0], 0.0f);
    const _Float16 b = (_Float16)__builtin_fmaf(p1, (float)as_h2(s1)[0], 0.0f);
    return h2_bits(half2_t{a, b});
}
// the fp16 of the remainders p0 * s0 - hi0 and p1 * s1 - hi1 (one fused multiply-add each)
__device__ __forceinline__ uint32_t pv_lo(float p0, uint32_t s0, float p1, uint32_t s1, uint32_t hi)
{
    const half2_t h = as_h2(hi);
    const _Float16 a = (_Float16)__builtin_fmaf(p0, (float)as_h2(s0)[0], -(float)h[0]);
    const _Float16 b = (_Float16)__builtin_fmaf(p1, (float)as_h2(s1)[0], -(float)h[1]);
    return h2_bits(half2_t{a, b});
}

// kernel arguments from the validated call arguments (host)
inline DecArgs make_dec_args(const DecodeParams &p)
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
    a.qnorm = p.qnorm;
    a.knew = p.knew;
    a.vnew = p.vnew;
    a.max_blocks = p.max_blocks;
    a.pool_blocks = p.pool_blocks;
    a.block_stride = p.block_stride;
    a.head_stride = p.head_stride;
    a.state = p.state;
    a.upd = p.upd;
    a.n_sink = p.n_sink;
    a.hybrid = p.hybrid;
    a.flag_off = p.flag_off;
    a.state_out = p.state_out;
    a.row_bytes = (int32_t)((int64_t)(p.n_packed / kBlockTokens) * p.block_bytes);
    a.out = p.out;
    a.out_f16 = p.out_f16;
    a.ws = p.ws;
    a.n_chunks = (a.gq + 3) / 4;
    a.rec_per_group = fused_records(p.num_splits);
    return a;
}

// token range of split `split` (the rule the header documents): packed tiles
// [tlo, thi) and whether the split also takes the fp16 window
__device__ __forceinline__ void split_range(const DecArgs &a, int split, int &tlo, int &thi,
                                            bool &with_res)
{
    const int NT = a.n_packed / kTile;
    tlo = 0;
    thi = 0;
    if (a.res_alone && split == a.S - 1) {
        with_res = true;
    } else {
        tlo = (int)((int64_t)split * NT / a.Sp);
        thi = (int)((int64_t)(split + 1) * NT / a.Sp);
        with_res = !a.res_alone && split == a.S - 1;
    }
    with_res = with_res && a.n_res > 0;
}

// The same rule for one sequence of a paged cache with its own lengths: NT = ceil(n / 32)
// tiles, the last one possibly partial.
__device__ __forceinline__ void split_range_seq(const DecArgs &a, int split, int n_packed,
                                                int n_res, int &tlo, int &thi, bool &with_res)
{
    const int NT = (n_packed + kTile - 1) / kTile;
    const bool res_alone = a.S > 1 && n_res > 0;
    const int Sp = res_alone ? a.S - 1 : a.S;
    tlo = 0;
    thi = 0;
    if (res_alone && split == a.S - 1) {
        with_res = true;
    } else {
        tlo = (int)((int64_t)split * NT / Sp);
        thi = (int)((int64_t)(split + 1) * NT / Sp);
        with_res = !res_alone && split == a.S - 1;
    }
    with_res = with_res && n_res > 0;
}

}  // namespace
}  // namespace kvq
