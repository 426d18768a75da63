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

// max / sum over the 16 lanes of a row; every lane of the row gets the result
__device__ __forceinline__ float row_max16(float v)
{
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0xB1>(v));
    return v;
}
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

// fp16 magic-number conversion of small integer codes: OR-ing a code into the low
// mantissa bits of a power of two 2^E gives the fp16 value 2^E + code * 2^(E-10+shift);
// subtracting 2^E (exact) leaves the code. Each pair below holds two codes in the two
// halves of a 32-bit word.
__device__ __forceinline__ half2_t magic_pair(uint32_t bits_in_place, uint32_t mask, uint32_t base_bits)
{
    const uint32_t u = (bits_in_place & mask) | base_bits;
    const _Float16 base = __builtin_bit_cast(_Float16, (uint16_t)(base_bits & 0xffff));
    return as_h2(u) - half2_t{base, base};
}

// Eight codes of one 8-channel octet -> half8 in the slot order (0,4,1,5,2,6,3,7):
// slot 2m holds channel m, slot 2m+1 holds channel m+4.
//  4-bit: the octet is a 32-bit word, code i at bits 4i.
__device__ __forceinline__ half8_t unpack_octet4(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    half2_t p0 = magic_pair(w, 0x000F000Fu, 0x64006400u);   // c0,c4   (2^10 + c)
    half2_t p1 = magic_pair(w, 0x00F000F0u, 0x54005400u);   // c1,c5   (2^6 + c)
    half2_t p2 = magic_pair(w8, 0x000F000Fu, 0x64006400u);  // c2,c6
    half2_t p3 = magic_pair(w8, 0x00F000F0u, 0x54005400u);  // c3,c7
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  2-bit: the octet is 16 bits (low half of y), code i at bits 2i.
__device__ __forceinline__ half8_t unpack_octet2(uint32_t y)
{
    // c0..c3 (byte 0) stay in bits 0-7; c4..c7 (byte 1) move to bits 16-23
    const uint32_t w = perm_b32(0u, y, 0x0c010c00u);
    half2_t p0 = magic_pair(w, 0x00030003u, 0x64006400u);   // 2^10 + c
    half2_t p1 = magic_pair(w, 0x000C000Cu, 0x5C005C00u);   // 2^8 + c
    half2_t p2 = magic_pair(w, 0x00300030u, 0x54005400u);   // 2^6 + c
    half2_t p3 = magic_pair(w, 0x00C000C0u, 0x4C004C00u);   // 2^4 + c
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
//  3-bit: the octet is 24 bits (low bits of x), code i at bits 3i.
__device__ __forceinline__ half8_t unpack_octet3(uint32_t x)
{
    // c0..c3 (bits 0-11) stay; c4..c7 (bits 12-23) move to bits 16-27
    const uint32_t w = __builtin_amdgcn_ubfe(x, 0, 12) | ((x << 4) & 0x0FFF0000u);
    half2_t p0 = magic_pair(w, 0x00070007u, 0x64006400u);        // 2^10 + c
    half2_t p1 = magic_pair(w, 0x00380038u, 0x58005800u);        // 2^7 + c
    half2_t p2 = magic_pair(w, 0x01C001C0u, 0x4C004C00u);        // 2^4 + c
    half2_t p3 = magic_pair(w >> 3, 0x01C001C0u, 0x4C004C00u);   // 2^4 + c
    return half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Two tokens' octets (a = token 2m, b = token 2m+1) -> for each channel c of the octet a
// half2 {code(a, c), code(b, c)}; out[c] for c = 0..7.
__device__ __forceinline__ void pair_tokens4(uint32_t a, uint32_t b, half2_t out[8])
{
    const uint32_t lo = pack_lo16(a, b);   // channels 0..3 of both tokens
    const uint32_t hi = pack_hi16(a, b);   // channels 4..7
    const uint32_t lo8 = lo >> 8, hi8 = hi >> 8;
    out[0] = magic_pair(lo, 0x000F000Fu, 0x64006400u);
    out[1] = magic_pair(lo, 0x00F000F0u, 0x54005400u);
    out[2] = magic_pair(lo8, 0x000F000Fu, 0x64006400u);
    out[3] = magic_pair(lo8, 0x00F000F0u, 0x54005400u);
    out[4] = magic_pair(hi, 0x000F000Fu, 0x64006400u);
    out[5] = magic_pair(hi, 0x00F000F0u, 0x54005400u);
    out[6] = magic_pair(hi8, 0x000F000Fu, 0x64006400u);
    out[7] = magic_pair(hi8, 0x00F000F0u, 0x54005400u);
}
__device__ __forceinline__ void pair_tokens2(uint32_t a, uint32_t b, half2_t out[8])
{
    const uint32_t u = pack_lo16(a, b);    // 16-bit octets side by side
    const uint32_t u8 = u >> 8;
    out[0] = magic_pair(u, 0x00030003u, 0x64006400u);
    out[1] = magic_pair(u, 0x000C000Cu, 0x5C005C00u);
    out[2] = magic_pair(u, 0x00300030u, 0x54005400u);
    out[3] = magic_pair(u, 0x00C000C0u, 0x4C004C00u);
    out[4] = magic_pair(u8, 0x00030003u, 0x64006400u);
    out[5] = magic_pair(u8, 0x000C000Cu, 0x5C005C00u);
    out[6] = magic_pair(u8, 0x00300030u, 0x54005400u);
    out[7] = magic_pair(u8, 0x00C000C0u, 0x4C004C00u);
}
__device__ __forceinline__ void pair_tokens3(uint32_t a, uint32_t b, half2_t out[8])
{
    // channels 0..3 (bits 0-11) of a in the low half, of b in the high half
    const uint32_t lo = (a & 0x0000FFFFu) | (b << 16);
    // channels 4..7 (bits 12-23)
    const uint32_t hi = ((a >> 12) & 0x0000FFFFu) | ((b << 4) & 0xFFFF0000u);
    out[0] = magic_pair(lo, 0x00070007u, 0x64006400u);
    out[1] = magic_pair(lo, 0x00380038u, 0x58005800u);
    out[2] = magic_pair(lo, 0x01C001C0u, 0x4C004C00u);
    out[3] = magic_pair(lo >> 3, 0x01C001C0u, 0x4C004C00u);
    out[4] = magic_pair(hi, 0x00070007u, 0x64006400u);
    out[5] = magic_pair(hi, 0x00380038u, 0x58005800u);
    out[6] = magic_pair(hi, 0x01C001C0u, 0x4C004C00u);
    out[7] = magic_pair(hi >> 3, 0x01C001C0u, 0x4C004C00u);
}

}  // namespace kvq
