// kvq_device.h -- device-side helpers shared by the libkvq HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kGroups = kHeadDim / kGroup;  // 4 groups per token
constexpr int kBlockTokens = 128;

// ---- DPP lane moves (wave64; rows are 16 lanes, quads 4 lanes) -------------------
// quad_perm encodings: xor 1 -> [1,0,3,2] = 0xB1, xor 2 -> [2,3,0,1] = 0x4E.
// row_ror:n = 0x120 + n rotates within each 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max over the 16 lanes of a row (finite values or -inf); every lane of the row gets the
// result. Each step is a DPP move and v_med3_f32 against FLT_MAX: the median of
// {a, b, FLT_MAX} is max(a, b). Built from compiler intrinsics rather than inline asm, so
// that the compiler sees every VGPR write and inserts the wait states that DPP and MFMA
// neighbours need.
template <int CTRL>
__device__ __forceinline__ float dpp_bc(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float v)
{
    constexpr float kBig = 3.402823466e38f;
    v = __builtin_amdgcn_fmed3f(v, dpp_bc<0x128>(v), kBig);
    v = __builtin_amdgcn_fmed3f(v, dpp_bc<0x124>(v), kBig);
    v = __builtin_amdgcn_fmed3f(v, dpp_bc<0x4E>(v), kBig);
    v = __builtin_amdgcn_fmed3f(v, dpp_bc<0xB1>(v), kBig);
    return v;
}
// sum over the 16 lanes of a row; every lane of the row gets the result
__device__ __forceinline__ float row_sum16(float v)
{
    v = v + dpp_f<0x128>(v);
    v = v + dpp_f<0x124>(v);
    v = v + dpp_f<0x4E>(v);
    v = v + dpp_f<0xB1>(v);
    return v;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// (lo & 0xffff) | (hi << 16)     and     (lo >> 16) | (hi & 0xffff0000)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x07060302u); }

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t h2_bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// A 32-bit constant held in a VGPR. The fp16 magic-number unpack below is
// (bits & mask) | base with two 32-bit constants; gfx9 VOP3 takes at most one SGPR
// operand, so keeping `base` in a VGPR lets the compiler fuse it into one v_and_or_b32.
__device__ __forceinline__ uint32_t vconst(uint32_t c)
{
    // an identity DPP move: a VALU op the compiler cannot fold back into a literal
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)c, 0xE4, 0xF, 0xF, false);
}

// fp16 magic-number conversion of small integer codes: OR-ing a code into the mantissa of
// 2^6 (0x5400), at bits 4.. where one unit of the code weighs exactly 1, gives the fp16
// value 64 + code exactly.
struct Magic {
    uint32_t b6;
    __device__ __forceinline__ Magic() : b6(vconst(0x54005400u)) {}
};

// two codes (one per 16-bit half) -> half2 of 2^E + code
__device__ __forceinline__ uint32_t mpair(uint32_t bits, uint32_t mask, uint32_t vbase)
{
    return (bits & mask) | vbase;
}

// Eight codes of one 8-channel octet -> half8 of 64 + code, in the slot order
// (0,4,1,5,2,6,3,7): slot 2m holds channel m, slot 2m+1 holds channel m+4 (used for K,
// where the query operand is laid out in the same order). Every code is moved to the bits
// whose weight at 2^6 is 1 (bits 4.. of each half), so all slots carry the same offset 64,
// which the caller removes exactly through the accumulator (-64 * sum of q).
//  4-bit: the octet is a 32-bit word, code i at bits 4i.
__device__ __forceinline__ half8_t unpack_octet4(uint32_t w, const Magic &M)
{
    const uint32_t m = 0x00F000F0u;
    const half2_t p0 = as_h2(mpair(w << 4, m, M.b6));   // c0,c4
    const half2_t p1 = as_h2(mpair(w, m, M.b6));        // c1,c5
    const half2_t p2 = as_h2(mpair(w >> 4, m, M.b6));   // c2,c6
    const half2_t p3 = as_h2(mpair(w >> 8, m, M.b6));   // c3,c7
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  2-bit: the octet is 16 bits (low half of y), code i at bits 2i.
__device__ __forceinline__ half8_t unpack_octet2(uint32_t y, const Magic &M)
{
    // c0..c3 (byte 0) stay in bits 0-7; c4..c7 (byte 1) move to bits 16-23
    const uint32_t w = perm_b32(0u, y, 0x0c010c00u);
    const uint32_t m = 0x00300030u;
    const half2_t p0 = as_h2(mpair(w << 4, m, M.b6));
    const half2_t p1 = as_h2(mpair(w << 2, m, M.b6));
    const half2_t p2 = as_h2(mpair(w, m, M.b6));
    const half2_t p3 = as_h2(mpair(w >> 2, m, M.b6));
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  3-bit: the octet is 24 bits (low bits of x), code i at bits 3i.
__device__ __forceinline__ half8_t unpack_octet3(uint32_t x, const Magic &M)
{
    // c0..c3 (bits 0-11) stay; c4..c7 (bits 12-23) move to bits 16-27
    const uint32_t w = pack_lo16(x, x >> 12);
    const uint32_t m = 0x00700070u;
    const half2_t p0 = as_h2(mpair(w << 4, m, M.b6));
    const half2_t p1 = as_h2(mpair(w << 1, m, M.b6));
    const half2_t p2 = as_h2(mpair(w >> 2, m, M.b6));
    const half2_t p3 = as_h2(mpair(w >> 5, m, M.b6));
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Two tokens' octets (a = token 2m, b = token 2m+1) -> for each channel c of the octet a
// half2 {64 + code(a, c), 64 + code(b, c)} (V operand; the 64 offset is removed through
// the zero-point term: zero' = zero - 64 * scale). Every code is first moved to the bit
// whose weight at 2^6 is 1 (bits 4.. of each half).
__device__ __forceinline__ void pair_tokens4(uint32_t a, uint32_t b, const Magic &M, half2_t out[8])
{
    const uint32_t lo = pack_lo16(a, b);   // channels 0..3 of both tokens
    const uint32_t hi = pack_hi16(a, b);   // channels 4..7
    const uint32_t m = 0x00F000F0u;
    out[0] = as_h2(mpair(lo << 4, m, M.b6));
    out[1] = as_h2(mpair(lo, m, M.b6));
    out[2] = as_h2(mpair(lo >> 4, m, M.b6));
    out[3] = as_h2(mpair(lo >> 8, m, M.b6));
    out[4] = as_h2(mpair(hi << 4, m, M.b6));
    out[5] = as_h2(mpair(hi, m, M.b6));
    out[6] = as_h2(mpair(hi >> 4, m, M.b6));
    out[7] = as_h2(mpair(hi >> 8, m, M.b6));
}
__device__ __forceinline__ void pair_tokens2(uint32_t a, uint32_t b, const Magic &M, half2_t out[8])
{
    const uint32_t u = pack_lo16(a, b);    // 16-bit octets side by side
    const uint32_t m = 0x00300030u;
    out[0] = as_h2(mpair(u << 4, m, M.b6));
    out[1] = as_h2(mpair(u << 2, m, M.b6));
    out[2] = as_h2(mpair(u, m, M.b6));
    out[3] = as_h2(mpair(u >> 2, m, M.b6));
    out[4] = as_h2(mpair(u >> 4, m, M.b6));
    out[5] = as_h2(mpair(u >> 6, m, M.b6));
    out[6] = as_h2(mpair(u >> 8, m, M.b6));
    out[7] = as_h2(mpair(u >> 10, m, M.b6));
}
__device__ __forceinline__ void pair_tokens3(uint32_t a, uint32_t b, const Magic &M, half2_t out[8])
{
    const uint32_t lo = pack_lo16(a, b);              // channels 0..3 (bits 0-11 of each)
    const uint32_t hi = pack_lo16(a >> 12, b >> 12);  // channels 4..7
    const uint32_t m = 0x00700070u;
    out[0] = as_h2(mpair(lo << 4, m, M.b6));
    out[1] = as_h2(mpair(lo << 1, m, M.b6));
    out[2] = as_h2(mpair(lo >> 2, m, M.b6));
    out[3] = as_h2(mpair(lo >> 5, m, M.b6));
    out[4] = as_h2(mpair(hi << 4, m, M.b6));
    out[5] = as_h2(mpair(hi << 1, m, M.b6));
    out[6] = as_h2(mpair(hi >> 2, m, M.b6));
    out[7] = as_h2(mpair(hi >> 5, m, M.b6));
}

// ---- codes as fp16 subnormals ---------------------------------------------------------
// With a zero exponent field, fp16 mantissa bits [k, k + b) holding a code c give the
// subnormal value c * 2^(k - 24), exactly, and the gfx950 matrix cores multiply subnormal
// fp16 operands at their value. So a pair of codes (one per 16-bit half) becomes an MFMA
// operand with a single mask: no offset to add and none to remove, as long as the code
// sits inside bits 0..9. Each slot pair then carries a power-of-two weight 2^k (in units
// of 2^-24) that the other operand or the accumulator divides out exactly.
//
// Key operand: eight codes of one channel octet, in the slot order (0,4,1,5,2,6,3,7) of the
// query operand; slot pair p holds channels p and p + 4 with weight 2^raw_key_shift<BITS>(p).
template <int BITS>
__device__ __forceinline__ constexpr int raw_key_shift(int p)
{
    return BITS == 4 ? (p & 1) * 4 : BITS == 2 ? 2 * p : (p == 0 ? 0 : p == 1 ? 3 : 6);
}
//  4-bit: the octet is a 32-bit word, code i at bits 4i
__device__ __forceinline__ half8_t raw_octet4(uint32_t w)
{
    const uint32_t t = w >> 8;
    const half2_t p0 = as_h2(w & 0x000F000Fu);   // c0,c4  x1
    const half2_t p1 = as_h2(w & 0x00F000F0u);   // c1,c5  x16
    const half2_t p2 = as_h2(t & 0x000F000Fu);   // c2,c6  x1
    const half2_t p3 = as_h2(t & 0x00F000F0u);   // c3,c7  x16
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  2-bit: the octet is 16 bits (low half of y), code i at bits 2i
__device__ __forceinline__ half8_t raw_octet2(uint32_t y)
{
    const uint32_t w = perm_b32(0u, y, 0x0c010c00u);   // byte 0 -> low half, byte 1 -> high
    const half2_t p0 = as_h2(w & 0x00030003u);   // c0,c4  x1
    const half2_t p1 = as_h2(w & 0x000C000Cu);   // c1,c5  x4
    const half2_t p2 = as_h2(w & 0x00300030u);   // c2,c6  x16
    const half2_t p3 = as_h2(w & 0x00C000C0u);   // c3,c7  x64
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  3-bit: the octet is 24 bits (low bits of x), code i at bits 3i
__device__ __forceinline__ half8_t raw_octet3(uint32_t x)
{
    const uint32_t w = pack_lo16(x, x >> 12);            // c0..c3 low half, c4..c7 high half
    const half2_t p0 = as_h2(w & 0x00070007u);           // c0,c4  x1
    const half2_t p1 = as_h2(w & 0x00380038u);           // c1,c5  x8
    const half2_t p2 = as_h2(w & 0x01C001C0u);           // c2,c6  x64
    const half2_t p3 = as_h2((w >> 3) & 0x01C001C0u);    // c3,c7  x64 (bits 9-11 -> 6-8)
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Value operand: for each channel c of the octet a half2 {code(a, c), code(b, c)} of two
// tokens' octets, with weight 2^raw_value_shift<BITS>(c).
template <int BITS>
__device__ __forceinline__ constexpr int raw_value_shift(int c)
{
    return BITS == 4 ? (c & 1) * 4
         : BITS == 2 ? (c < 5 ? 2 * c : 2 * c - 6)
                     : ((c & 3) == 0 ? 0 : (c & 3) == 1 ? 3 : 6);
}
__device__ __forceinline__ void raw_pair4(uint32_t a, uint32_t b, half2_t out[8])
{
    const uint32_t lo = pack_lo16(a, b);   // channels 0..3 of both tokens
    const uint32_t hi = pack_hi16(a, b);   // channels 4..7
    const uint32_t lt = lo >> 8, ht = hi >> 8;
    out[0] = as_h2(lo & 0x000F000Fu);
    out[1] = as_h2(lo & 0x00F000F0u);
    out[2] = as_h2(lt & 0x000F000Fu);
    out[3] = as_h2(lt & 0x00F000F0u);
    out[4] = as_h2(hi & 0x000F000Fu);
    out[5] = as_h2(hi & 0x00F000F0u);
    out[6] = as_h2(ht & 0x000F000Fu);
    out[7] = as_h2(ht & 0x00F000F0u);
}
__device__ __forceinline__ void raw_pair2(uint32_t a, uint32_t b, half2_t out[8])
{
    const uint32_t u = pack_lo16(a, b);    // 16-bit octets side by side
    const uint32_t t = u >> 6;             // channels 5..7 (bits 10-15) -> bits 4-9
    out[0] = as_h2(u & 0x00030003u);
    out[1] = as_h2(u & 0x000C000Cu);
    out[2] = as_h2(u & 0x00300030u);
    out[3] = as_h2(u & 0x00C000C0u);
    out[4] = as_h2(u & 0x03000300u);
    out[5] = as_h2(t & 0x00300030u);
    out[6] = as_h2(t & 0x00C000C0u);
    out[7] = as_h2(t & 0x03000300u);
}
__device__ __forceinline__ void raw_pair3(uint32_t a, uint32_t b, half2_t out[8])
{
    const uint32_t lo = pack_lo16(a, b);              // channels 0..3 (bits 0-11 of each)
    const uint32_t hi = pack_lo16(a >> 12, b >> 12);  // channels 4..7
    const uint32_t lt = lo >> 3, ht = hi >> 3;
    out[0] = as_h2(lo & 0x00070007u);
    out[1] = as_h2(lo & 0x00380038u);
    out[2] = as_h2(lo & 0x01C001C0u);
    out[3] = as_h2(lt & 0x01C001C0u);
    out[4] = as_h2(hi & 0x00070007u);
    out[5] = as_h2(hi & 0x00380038u);
    out[6] = as_h2(hi & 0x01C001C0u);
    out[7] = as_h2(ht & 0x01C001C0u);
}

}  // namespace kvq
