// quant_common.h -- the group quantizer of one token's 32-channel group, held by a quad of
// lanes, shared by the block packer (quant_pack.hip) and the token-wise paged packers
// (paged.hip). BitDecoding page ("Tensor Core加速的低比特KV缓存解码系统") sec. 2.1 for
// scale = (max - min) / (2^b - 1) and code = round((x - min) / scale) with a cross-lane
// min/max (sec. 3.1); 3-bit blog page sec. 2.3 for the clip; InnerQ page
// ("KV缓存量化技术InnerQ：提升大模型推理效率") sec. 2.2 for the symmetric/asymmetric choice.
// The scales come from IEEE binary32 operations (no contraction; division correctly
// rounded), and every code equals the one the correctly rounded quotient (x - zero) / scale
// gives (see code_from_reciprocal), so the bytes equal the CPU definition's.
#pragma once

#include "kvq_device.h"

namespace kvq {
namespace {

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) { return dpp_f<CTRL>(v); }

__device__ __forceinline__ float round_half_away_pos(float t)
{
#pragma clang fp contract(off)
    const float k = __builtin_truncf(t);
    return (t - k >= 0.5f) ? k + 1.0f : k;
}
__device__ __forceinline__ float round_half_away(float t)
{
#pragma clang fp contract(off)
    const float r = round_half_away_pos(__builtin_fabsf(t));
    return t < 0.0f ? -r : r;
}

// round_half_away_pos(d / s) for d >= 0, s > 0, computed from r = rcp(s) instead of the
// correctly rounded division (which costs ~10 instructions and a branch per element).
// v_rcp_f32 is within 1 ulp of 1/s and the product adds half an ulp, so q = d * r differs
// from the correctly rounded quotient t by at most 2^-22 * q. The candidate c = floor(q +
// 1/2) is accepted when |q - c| < 1/2 - 2^-19 * q: then |t - c| < 1/2, so t rounds to c
// (whatever rounding q + 1/2 took). q - c is exact (Sterbenz for c >= 1; q itself for
// c = 0); the threshold's own rounding (<= 2^-26) stays inside the margin for q >= 2^-4 / 7,
// and below that c = 0 = round(t) anyway. Otherwise `near` is set and the caller redoes the
// element with the exact division. s == 0 is passed as r = 0 and yields 0, not near.
__device__ __forceinline__ float code_from_reciprocal(float d, float r, bool &near)
{
#pragma clang fp contract(off)
    const float q = d * r;
    const float c = __builtin_floorf(q + 0.5f);
    near = __builtin_fabsf(q - c) >= __builtin_fmaf(q, -0x1p-19f, 0.5f);
    return c;
}

// Quantize the group whose 32 fp16 values are spread over a DPP quad (lane j of the quad
// holds channels 8j .. 8j+7 in `raw`); every lane of the quad must be active. Returns this
// lane's 8 codes packed LSB-first (BITS bytes in the low bits of `packed`), the group's
// fp16 scale and zero, and its flag (1 asymmetric, 0 symmetric; always 1 without HYBRID).
template <int BITS, bool HYBRID>
__device__ __forceinline__ void quantize_octet(const u32x4 raw, uint32_t &packed,
                                               uint16_t &out_s, uint16_t &out_z, int &flag)
{
#pragma clang fp contract(off)
    constexpr int N = (1 << BITS) - 1;
    constexpr int OFF = 1 << (BITS - 1);
    constexpr int QS = OFF - 1;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = as_h2(raw[i]);
        x[2 * i] = (float)h.x;
        x[2 * i + 1] = (float)h.y;
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    mn = fminf(mn, quad_dpp<0xB1>(mn));
    mn = fminf(mn, quad_dpp<0x4E>(mn));
    mx = fmaxf(mx, quad_dpp<0xB1>(mx));
    mx = fmaxf(mx, quad_dpp<0x4E>(mx));
    mn = mn + 0.0f;   // -0.0 -> +0.0
    mx = mx + 0.0f;

    // asymmetric candidate
    const _Float16 sh = (_Float16)((mx - mn) / (float)N);
    const _Float16 zh = (_Float16)mn;     // exact
    const float s = (float)sh, z = (float)zh;
    int code[8];
    {
        const float rs = s != 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
        uint32_t near = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bool nr;
            code[i] = (int)fminf(code_from_reciprocal(x[i] - z, rs, nr), (float)N);
            near |= (uint32_t)nr << i;
        }
        // near a rounding boundary: the correctly rounded quotient decides (rare; a
        // wave-uniform branch)
        if (__builtin_amdgcn_ballot_w64(near != 0) != 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((near >> i) & 1u)
                    code[i] = (int)fminf(round_half_away_pos((x[i] - z) / s), (float)N);
        }
    }
    out_s = __builtin_bit_cast(uint16_t, sh);
    out_z = __builtin_bit_cast(uint16_t, zh);
    flag = 1;

    if (HYBRID) {
        // symmetric candidate: signed grid k*ss, |k| <= QS, offset-binary codes
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(x[i]));
        am = fmaxf(am, quad_dpp<0xB1>(am));
        am = fmaxf(am, quad_dpp<0x4E>(am));
        const _Float16 ssh = (_Float16)(am / (float)QS);
        const float ss = (float)ssh;
        const float zs = -((float)OFF * ss) + 0.0f;
        const bool eligible = __builtin_fabsf(zs) <= 65504.0f;
        // k = clamp(round_half_away(x / ss), -QS, QS) = sign(x) * min(QS, round(|x| / ss)),
        // from the reciprocal as above
        int scode[8];
        {
            const float rss = ss != 0.0f ? __builtin_amdgcn_rcpf(ss) : 0.0f;
            uint32_t near = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bool nr;
                const float k = fminf(code_from_reciprocal(__builtin_fabsf(x[i]), rss, nr), (float)QS);
                scode[i] = OFF + (int)(x[i] < 0.0f ? -k : k);
                near |= (uint32_t)nr << i;
            }
            if (__builtin_amdgcn_ballot_w64(near != 0) != 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((near >> i) & 1u)
                        scode[i] = OFF + (int)fminf(fmaxf(round_half_away(x[i] / ss), -(float)QS),
                                                    (float)QS);
            }
        }
        // squared errors, balanced pairwise sum in channel order: 8 in-lane, then quad
        float ea[8], es[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float da = x[i] - __builtin_fmaf((float)code[i], s, z);
            const float ds = x[i] - __builtin_fmaf((float)scode[i], ss, zs);
            ea[i] = da * da;
            es[i] = ds * ds;
        }
        float sa = ((ea[0] + ea[1]) + (ea[2] + ea[3])) + ((ea[4] + ea[5]) + (ea[6] + ea[7]));
        float se = ((es[0] + es[1]) + (es[2] + es[3])) + ((es[4] + es[5]) + (es[6] + es[7]));
        sa = sa + quad_dpp<0xB1>(sa);
        sa = sa + quad_dpp<0x4E>(sa);
        se = se + quad_dpp<0xB1>(se);
        se = se + quad_dpp<0x4E>(se);
        if (eligible && se < sa) {
            flag = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) code[i] = scode[i];
            out_s = __builtin_bit_cast(uint16_t, ssh);
            out_z = __builtin_bit_cast(uint16_t, (_Float16)zs);
        }
    }

    packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= (uint32_t)code[i] << (BITS * i);
}

}  // namespace
}  // namespace kvq
