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

struct DecArgs {
    const uint16_t *q;
    int32_t Hq, Hkv, gq, head_base;
    const uint8_t *kp, *vp;
    int64_t row_stride;
    int32_t n_packed;
    const uint16_t *kres, *vres;
    int32_t res_cap, n_res;
    float sm_log2;               // sm_scale * log2(e): logits are kept in the exp2 domain
    int32_t S, Sp, res_alone;
    float *part_o, *part_lse;
    int32_t block_bytes, sz_off;
};

struct Smem {
    float p[kWaves][4][kTile];   // p of head h, token t of the current tile
    float sv[kWaves][4][kTile];  // V scale of group g, token t
    float qs[4][4];              // sum of q over group g, head h
    float mo[kWaves][4][kHeadDim];
    float ml[kWaves][4][2];
};

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

template <int BITS>
struct KGroup;   // one token's 32-channel group of K codes

template <>
struct KGroup<4> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint8_t *p) { w = *reinterpret_cast<const u32x4 *>(p); }
    __device__ __forceinline__ half8_t octet(int o) const { return unpack_octet4(w[o]); }
};
template <>
struct KGroup<2> {
    u32x2 w;
    __device__ __forceinline__ void load(const uint8_t *p) { w = *reinterpret_cast<const u32x2 *>(p); }
    __device__ __forceinline__ half8_t octet(int o) const
    {
        return unpack_octet2((o & 1) ? (w[o >> 1] >> 16) : w[o >> 1]);
    }
};
template <>
struct KGroup<3> {
    uint32_t w0, w1, w2;
    __device__ __forceinline__ void load(const uint8_t *p)
    {
        const uint32_t *d = reinterpret_cast<const uint32_t *>(p);
        w0 = d[0];
        w1 = d[1];
        w2 = d[2];
    }
    __device__ __forceinline__ half8_t octet(int o) const
    {
        uint32_t x = o == 0 ? w0 : o == 1 ? __builtin_amdgcn_alignbit(w1, w0, 24)
                               : o == 2 ? __builtin_amdgcn_alignbit(w2, w1, 16) : (w2 >> 8);
        return unpack_octet3(x);
    }
};

// V codes of channel octet j of one token (low bits of the result)
template <int BITS>
__device__ __forceinline__ uint32_t load_v_octet(const uint8_t *tok_row, int j)
{
    if (BITS == 4) return reinterpret_cast<const uint32_t *>(tok_row)[j];
    if (BITS == 2) return reinterpret_cast<const uint16_t *>(tok_row)[j];
    // 3 bits: bytes 3j..3j+2 of the 48-byte row; read the two dwords that cover them.
    // For j = 15 the second dword is the next 4 bytes of the block (next token's codes,
    // or the first scale/zero bytes after token 127), always inside the block.
    const int byte = 3 * j;
    const uint32_t *d = reinterpret_cast<const uint32_t *>(tok_row + (byte & ~3));
    return __builtin_amdgcn_alignbit(d[1], d[0], (byte & 3) * 8);
}

template <int BITS>
__device__ __forceinline__ void pair_tokens(uint32_t a, uint32_t b, half2_t out[8])
{
    if (BITS == 4) pair_tokens4(a, b, out);
    else if (BITS == 2) pair_tokens2(a, b, out);
    else pair_tokens3(a, b, out);
}

__device__ __forceinline__ float sel4(const float4_t &v, int k)
{
    return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3];
}

// Softmax update and PV for one 32-token tile whose logits (exp2 domain) are lg[0]
// (token n) and lg[1] (token 16 + n), the V B-operand pairs vpair[m][c] (tokens 8r+2m,
// 8r+2m+1 of the tile, channel c of octet n), and the per-token V scale of group r
// already written to LDS by this lane.
template <int NH>
__device__ __forceinline__ void softmax_pv(Smem &sm, int wave, int n, int r, const float lg[2],
                                           const float zv[2][4], const half2_t vpair[4][8],
                                           float &m, float &l, float zacc[4], float4_t dpv[8])
{
    float tmax = row_max16(fmaxf(lg[0], lg[1]));
    const float mnew = fmaxf(m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    const float p0 = __builtin_amdgcn_exp2f(lg[0] - mnew);
    const float p1 = __builtin_amdgcn_exp2f(lg[1] - mnew);
    m = mnew;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
        l *= alpha;
#pragma unroll
        for (int g = 0; g < 4; ++g) zacc[g] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) dpv[c] *= alpha;
    }
    l += p0 + p1;
#pragma unroll
    for (int g = 0; g < 4; ++g) zacc[g] += p0 * zv[0][g] + p1 * zv[1][g];

    sm.p[wave][r][n] = p0;
    sm.p[wave][r][16 + n] = p1;
    lds_fence();

    // A operand of PV: lane (i, r) holds rows i = 4h + g, token slots 8r .. 8r+7
    const int i = n;
    const int hA = i >> 2, gA = i & 3;
    const float4_t pl = *reinterpret_cast<const float4_t *>(&sm.p[wave][hA][8 * r]);
    const float4_t ph = *reinterpret_cast<const float4_t *>(&sm.p[wave][hA][8 * r + 4]);
    const float4_t sl = *reinterpret_cast<const float4_t *>(&sm.sv[wave][gA][8 * r]);
    const float4_t sh = *reinterpret_cast<const float4_t *>(&sm.sv[wave][gA][8 * r + 4]);
    float w[8] = {pl[0] * sl[0], pl[1] * sl[1], pl[2] * sl[2], pl[3] * sl[3],
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
        dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, dpv[c], 0, 0, 0);
        dpv[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, dpv[c], 0, 0, 0);
    }
    // the next tile rewrites sm.p / sm.sv only after these reads have returned
    lds_fence();
}

template <int BITS, int NH>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a)
{
    __shared__ Smem sm;
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

    // ---- q: per-group sums (wave 0) and the QK A operands (every wave) ----
    const uint16_t *qb = a.q + ((int64_t)b * a.Hq + h0) * kHeadDim;
    if (wave == 0) {
        const int hh = lane >> 4, gg = (lane >> 2) & 3, qq = lane & 3;
        float s = 0.0f;
        if (hh < NH) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qb + hh * kHeadDim + gg * 32 + qq * 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const half2_t hv = as_h2(v[k]);
                s += (float)hv.x + (float)hv.y;
            }
        }
        s += dpp_f<0xB1>(s);
        s += dpp_f<0x4E>(s);
        if (qq == 0) sm.qs[hh][gg] = s;
    }
    half8_t aq[4];
    {
        const int hA = n >> 2, gA = n & 3;
        const bool live = (gA == r) && (hA < NH);
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            half8_t v = {};
            if (live) v = perm_octet_f16(*reinterpret_cast<const u32x4 *>(qb + hA * kHeadDim + 32 * r + 8 * o));
            aq[o] = v;
        }
    }
    __syncthreads();
    float qs[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) qs[g] = sm.qs[r][g];

    float m = -INFINITY, l = 0.0f;
    float zacc[4] = {0.f, 0.f, 0.f, 0.f};
    float4_t dpv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) dpv[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    const uint8_t *krow = a.kp + row * a.row_stride;
    const uint8_t *vrow = a.vp + row * a.row_stride;
    constexpr int TOKB = kHeadDim * BITS / 8;       // code bytes per token
    constexpr int GB = 4 * BITS;                    // code bytes per group

    // ---- packed tiles ----
    for (int t = tlo + wave; t < thi; t += kWaves) {
        const int tok0 = t * kTile;
        const uint8_t *kb = krow + (int64_t)(tok0 >> 7) * a.block_bytes;
        const uint8_t *vb = vrow + (int64_t)(tok0 >> 7) * a.block_bytes;
        const int tb0 = tok0 & 127;

        KGroup<BITS> kc[2];
        u32x4 ksz[2], vsz[2];
        uint32_t vc[8];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tb = tb0 + 16 * u + n;
            kc[u].load(kb + tb * TOKB + r * GB);
            ksz[u] = *reinterpret_cast<const u32x4 *>(kb + a.sz_off + tb * 16);
            vsz[u] = *reinterpret_cast<const u32x4 *>(vb + a.sz_off + tb * 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) vc[e] = load_v_octet<BITS>(vb + (tb0 + 8 * r + e) * TOKB, n);

        float lg[2], zv[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int o = 0; o < 4; ++o)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[o], kc[u].octet(o), acc, 0, 0, 0);
            float s = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const half2_t szk = as_h2(ksz[u][g]);
                s = __builtin_fmaf((float)szk.x, acc[g], s);
                s = __builtin_fmaf((float)szk.y, qs[g], s);
                const half2_t szv = as_h2(vsz[u][g]);
                zv[u][g] = (float)szv.y;
            }
            lg[u] = s * a.sm_log2;
            sm.sv[wave][r][16 * u + n] = (float)as_h2(vsz[u][r]).x;
        }
        half2_t vpair[4][8];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) pair_tokens<BITS>(vc[2 * mm], vc[2 * mm + 1], vpair[mm]);
        softmax_pv<NH>(sm, wave, n, r, lg, zv, vpair, m, l, zacc, dpv);
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
                sm.sv[wave][r][16 * u + n] = 1.0f;
            }
            u32x4 vt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ts = rt * kTile + 8 * r + e;
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
            softmax_pv<NH>(sm, wave, n, r, lg, zv, vpair, m, l, zacc, dpv);
        }
    }

    // ---- merge the waves ----
    const float lsum = row_sum16(l);
    float zr[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) zr[g] = row_sum16(zacc[g]);
    {
        const int gj = n >> 2;   // group of channels 8n .. 8n+7
        const float zg = sel4(float4_t{zr[0], zr[1], zr[2], zr[3]}, gj);
        float4_t o0, o1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0[c] = sel4(dpv[c], gj) + zg;
            o1[c] = sel4(dpv[4 + c], gj) + zg;
        }
        *reinterpret_cast<float4_t *>(&sm.mo[wave][r][8 * n]) = o0;
        *reinterpret_cast<float4_t *>(&sm.mo[wave][r][8 * n + 4]) = o1;
        if (n == 0) {
            sm.ml[wave][r][0] = m;
            sm.ml[wave][r][1] = lsum;
        }
    }
    __syncthreads();
    {
        const int h = threadIdx.x >> 6;       // 4 heads x 64 threads x 2 channels
        const int d = (threadIdx.x & 63) * 2;
        if (h < NH) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.ml[w][h][0]);
            float o0 = 0.f, o1 = 0.f, L = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float e = __builtin_amdgcn_exp2f(sm.ml[w][h][0] - M);
                    L += e * sm.ml[w][h][1];
                    o0 += e * sm.mo[w][h][d];
                    o1 += e * sm.mo[w][h][d + 1];
                }
            }
            const int64_t hq = (int64_t)b * a.Hq + h0 + h;
            const int64_t ob = (hq * a.S + split) * kHeadDim + d;
            if (L > 0.f) {
                const float inv = 1.0f / L;
                a.part_o[ob] = o0 * inv;
                a.part_o[ob + 1] = o1 * inv;
                if (d == 0) a.part_lse[hq * a.S + split] = (M + __log2f(L)) * 0.69314718055994531f;
            } else {
                a.part_o[ob] = 0.f;
                a.part_o[ob + 1] = 0.f;
                if (d == 0) a.part_lse[hq * a.S + split] = -INFINITY;
            }
        }
    }
}

template <int BITS, int NH>
hipError_t launch_t(const DecArgs &a, int64_t rows, int chunks, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_kernel<BITS, NH>), dim3((uint32_t)rows, (uint32_t)a.S, (uint32_t)chunks),
                       dim3(256), 0, stream, a);
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
