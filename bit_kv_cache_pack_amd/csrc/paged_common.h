// paged_common.h -- writing one quantized token into a paged packed cache (device side),
// shared by the cache-update kernels and the decode that folds the update in.
//
// Packed token j of sequence b, kv-head h: pool block tbl[b][j / 128] at
// pool + blk * block_stride + h * head_stride, token j % 128 inside the block. A table
// entry outside [0, pool_blocks) or a position beyond the table is skipped (nothing is
// written), so a wrong table can give wrong results but never an access outside the pool.
#pragma once

#include "kvq_device.h"

namespace kvq {

struct PoolGeom {
    uint8_t *pool;
    int64_t pool_blocks, block_stride, head_stride;
    const int32_t *tbl;
    int32_t max_blocks;
    int32_t sz_off, flag_off;
};

// Block that holds packed position j of (b, h), or null when the table does not map it.
__device__ __forceinline__ uint8_t *block_of(const PoolGeom &g, int b, int h, int64_t j)
{
    const int64_t e = j >> 7;
    if (j < 0 || e >= g.max_blocks) return nullptr;
    const int64_t blk = g.tbl[(int64_t)b * g.max_blocks + e];
    if (blk < 0 || blk >= g.pool_blocks) return nullptr;
    return g.pool + blk * g.block_stride + (int64_t)h * g.head_stride;
}

// Store one lane's share of token tb of a block: its code bytes, and (lane 0 of the
// quad) the group's scale/zero and flag bit.
template <int BITS, bool HYBRID>
__device__ __forceinline__ void store_octet(uint8_t *blk, const PoolGeom &g, int tb, int oct,
                                            uint32_t packed, uint16_t s, uint16_t z, int flag)
{
    constexpr int GBYTES = 4 * BITS;
    const int grp = oct >> 2, jq = oct & 3;
    uint8_t *gptr = blk + (tb * kGroups + grp) * GBYTES + jq * BITS;
    if (BITS == 4) {
        *reinterpret_cast<uint32_t *>(gptr) = packed;
    } else if (BITS == 2) {
        *reinterpret_cast<uint16_t *>(gptr) = (uint16_t)packed;
    } else {
        gptr[0] = (uint8_t)packed;
        gptr[1] = (uint8_t)(packed >> 8);
        gptr[2] = (uint8_t)(packed >> 16);
    }
    if (jq == 0) {
        *reinterpret_cast<uint32_t *>(blk + g.sz_off + (tb * kGroups + grp) * 4) =
            (uint32_t)s | ((uint32_t)z << 16);
        if (HYBRID) {
            // other tokens of the same 32-bit flag word may be written at the same time:
            // clear and set this group's bit with atomics that touch no other bit
            const int bit = tb * kGroups + grp;
            uint32_t *w = reinterpret_cast<uint32_t *>(blk + g.flag_off) + (bit >> 5);
            atomicAnd(w, ~(1u << (bit & 31)));
            if (flag) atomicOr(w, 1u << (bit & 31));
        }
    }
}

}  // namespace kvq
