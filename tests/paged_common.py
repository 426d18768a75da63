"""Helpers for the paged-cache tests: seeded block tables, pools and sequence states, and
a reader of one token's fields (codes, scale/zero, flag bits) in a packed block. No
quantization or attention arithmetic here."""
from __future__ import annotations

import numpy as np

SENTINEL = 0xA5


def make_table(rng, B: int, blocks_per_seq, n_pool_blocks: int | None = None):
    """A block table [B][max_blocks] whose used entries are distinct pool blocks in a random
    order (unused entries -1), and the pool size."""
    blocks_per_seq = list(blocks_per_seq)
    need = sum(blocks_per_seq)
    n_pool = max(need, 1) if n_pool_blocks is None else n_pool_blocks
    perm = rng.permutation(n_pool)[:need]
    maxb = max(max(blocks_per_seq), 1)
    tbl = np.full((B, maxb), -1, np.int32)
    k = 0
    for b, nb in enumerate(blocks_per_seq):
        tbl[b, :nb] = perm[k:k + nb]
        k += nb
    return tbl, n_pool


def new_pool(n_blocks: int, Hkv: int, block_bytes: int, fill: int = SENTINEL):
    return np.full((n_blocks, Hkv, block_bytes), fill, np.uint8)


def token_fields(fmt, block: np.ndarray, t: int):
    """(codes bytes, scale/zero bytes, flag bits) of token t of one packed block."""
    ng = fmt.head_dim // 32
    gb = 4 * fmt.bits
    codes = block[t * ng * gb:(t + 1) * ng * gb]
    sz = block[fmt.sz_offset + t * ng * 4: fmt.sz_offset + (t + 1) * ng * 4]
    if fmt.hybrid:
        bits = [(int(block[fmt.flag_offset + (t * ng + g) // 8]) >> ((t * ng + g) % 8)) & 1
                for g in range(ng)]
    else:
        bits = []
    return codes.copy(), sz.copy(), bits


def blocks_for(n_tokens: int) -> int:
    return (n_tokens + 127) // 128
