"""Pins of the oracle's paged cache, ragged lengths and per-token sliding window (InnerQ
page sec. 2.3; 3-bit blog page sec. 6.1).

- token-wise packing into table-addressed pool blocks gives the same bytes as the (pinned)
  block quantizer, and touches nothing else;
- a run of append/evict steps keeps the sinks, keeps the most recent tokens in the window
  and packs the others in arrival order, each with the block quantizer's bytes;
- attention over a paged cache equals the (pinned) contiguous attention when the pages are
  a permutation of a contiguous cache; a ragged tail of packed tokens equals the same
  values held in the fp16 window (exact-grid data, so dequantization is exact);
- bytes past a sequence's length never matter; split partials merge to the one-pass result.
"""
import numpy as np
import pytest

import paged_common as P

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _grid_tokens(rng, n_rows, T, bits):
    """fp16 tokens whose every 32-channel group is zero + c/16 with c covering 0..2^b-1:
    the asymmetric quantizer stores scale 1/16 and these codes, and decodes them exactly."""
    N = (1 << bits) - 1
    c = rng.integers(0, N + 1, (n_rows, T, 4, 32))
    c[..., 0] = 0
    c[..., 1] = N
    m = rng.integers(-40, 40, (n_rows, T, 4, 1)) / 16.0
    return _f16((m + c / 16.0).reshape(n_rows, T, 128))


@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, False), (2, True), (3, True)])
def test_token_packing_equals_block_quantizer(oracle_mod, bits, hybrid):
    O = oracle_mod
    rng = np.random.default_rng(bits + 10 * hybrid)
    fmt = O.Format(bits, 128, hybrid)
    B, Hkv, T = 2, 3, 256
    src = _f16(rng.standard_normal((B * Hkv, T, 128)) * rng.uniform(0.1, 4, (B * Hkv, 1, 128)))
    tbl, npool = P.make_table(rng, B, [2, 2], n_pool_blocks=7)
    pool = P.new_pool(npool, Hkv, fmt.block_bytes)
    O.pack_tokens_paged(fmt, src, B, Hkv, [T, T], [0, 0], pool, tbl)
    ref = O.quantize_pack(fmt, src)                        # contiguous rows of 2 blocks
    bb = fmt.block_bytes
    used = set()
    for b in range(B):
        for h in range(Hkv):
            for j in range(2):
                blk = tbl[b, j]
                used.add(int(blk))
                assert np.array_equal(pool[blk, h], ref[b * Hkv + h, j * bb:(j + 1) * bb])
    for blk in set(range(npool)) - used:
        assert np.all(pool[blk] == P.SENTINEL)


@pytest.mark.parametrize("bits,hybrid", [(4, False), (2, True)])
def test_ragged_token_packing_writes_only_its_tokens(oracle_mod, bits, hybrid):
    O = oracle_mod
    rng = np.random.default_rng(5)
    fmt = O.Format(bits, 128, hybrid)
    B, Hkv, T = 3, 2, 300
    count, start = [37, 0, 200], [5, 0, 130]
    src = _f16(rng.standard_normal((B * Hkv, T, 128)) * 2)
    tbl, npool = P.make_table(rng, B, [1, 1, 3])
    pool = P.new_pool(npool, Hkv, fmt.block_bytes)
    O.pack_tokens_paged(fmt, src, B, Hkv, count, start, pool, tbl)
    sentinel_block = P.new_pool(1, 1, fmt.block_bytes)[0, 0]
    for b in range(B):
        for h in range(Hkv):
            # the block quantizer's bytes of these tokens, at their positions
            ref = np.zeros((T + 512, 128), np.float16)
            ref[start[b]:start[b] + count[b]] = src[b * Hkv + h, :count[b]]
            nb = (start[b] + count[b] + 127) // 128 if count[b] else 0
            refp = O.quantize_pack(fmt, ref[None, :max(nb, 1) * 128])[0] if nb else None
            for j in range(tbl.shape[1]):
                if tbl[b, j] < 0:
                    continue
                blk = pool[tbl[b, j], h]
                for t in range(128):
                    pos = j * 128 + t
                    got = P.token_fields(fmt, blk, t)
                    if start[b] <= pos < start[b] + count[b]:
                        want = P.token_fields(fmt, refp[j * fmt.block_bytes:(j + 1) * fmt.block_bytes], t)
                    else:
                        want = P.token_fields(fmt, sentinel_block, t)
                    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
                    assert got[2] == want[2]


def _window_identity(win_k, b, h, slot):
    """Each test token carries its arrival index in channel 0 (exact in fp16)."""
    return int(win_k[b, h, slot, 0])


@pytest.mark.parametrize("bits,hybrid,cap,n_sink", [(4, False, 16, 4), (3, True, 8, 0),
                                                     (2, False, 5, 1)])
def test_append_evict_keeps_sinks_recent_and_arrival_order(oracle_mod, bits, hybrid, cap,
                                                            n_sink):
    O = oracle_mod
    rng = np.random.default_rng(cap)
    fmt = O.Format(bits, 128, hybrid)
    B, Hkv = 3, 2
    steps = 300
    # token i of sequence b (i counts from 0 over the whole run, prefill included)
    n_pre = [0, cap, 3]                     # tokens already in each window
    total = [n_pre[b] + steps for b in range(B)]
    toks_k = _f16(rng.standard_normal((B, Hkv, max(total), 128)))
    toks_v = _f16(rng.standard_normal((B, Hkv, max(total), 128)))
    toks_k[..., 0] = np.arange(max(total))[None, None, :]      # identity tag
    max_packed = max(total)
    tbl, npool = P.make_table(rng, B, [P.blocks_for(max_packed)] * B)
    kpool = P.new_pool(npool, Hkv, fmt.block_bytes)
    vpool = P.new_pool(npool, Hkv, fmt.block_bytes)
    kres = np.zeros((B, Hkv, cap, 128), np.float16)
    vres = np.zeros_like(kres)
    state = np.zeros((B, 4), np.int32)
    for b in range(B):
        kres[b, :, :n_pre[b]] = toks_k[b, :, :n_pre[b]]
        vres[b, :, :n_pre[b]] = toks_v[b, :, :n_pre[b]]
        state[b] = [0, n_pre[b], n_sink, 0]
    for i in range(steps):
        kn = np.stack([toks_k[b, :, n_pre[b] + i] for b in range(B)])
        vn = np.stack([toks_v[b, :, n_pre[b] + i] for b in range(B)])
        O.append_evict(fmt, kn, vn, kres, vres, n_sink, kpool, vpool, tbl, state)
    for b in range(B):
        n_all = total[b]
        n_packed = n_all - cap
        assert state[b, 0] == n_packed and state[b, 1] == cap
        assert n_sink <= state[b, 2] < cap
        for h in range(Hkv):
            ids = sorted(_window_identity(kres, b, h, s) for s in range(cap))
            sinks = [_window_identity(kres, b, h, s) for s in range(n_sink)]
            # sinks are the first n_sink tokens, the rest of the window the newest ones
            assert sinks == list(range(n_sink))
            assert ids == list(range(n_sink)) + list(range(n_all - (cap - n_sink), n_all))
            # packed position j holds token n_sink + j (arrival order), quantized as a block
            # quantizer quantizes it
            order = np.arange(n_sink, n_sink + n_packed)
            ref = O.quantize_pack(fmt, np.concatenate(
                [toks_k[b, h, order], np.zeros((P.blocks_for(n_packed) * 128 - n_packed, 128),
                                               np.float16)])[None])[0]
            refv = O.quantize_pack(fmt, np.concatenate(
                [toks_v[b, h, order], np.zeros((P.blocks_for(n_packed) * 128 - n_packed, 128),
                                               np.float16)])[None])[0]
            bb = fmt.block_bytes
            for j in range(n_packed):
                blk, t = tbl[b, j // 128], j % 128
                for pool, r in ((kpool, ref), (vpool, refv)):
                    got = P.token_fields(fmt, pool[blk, h], t)
                    want = P.token_fields(fmt, r[(j // 128) * bb:(j // 128 + 1) * bb], t)
                    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
                    assert got[2] == want[2]
            # and the window values are exactly the tokens (fp16 kept as is)
            for s in range(cap):
                tid = _window_identity(kres, b, h, s)
                assert np.array_equal(kres[b, h, s].view(np.uint16), toks_k[b, h, tid].view(np.uint16))
                assert np.array_equal(vres[b, h, s].view(np.uint16), toks_v[b, h, tid].view(np.uint16))


@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, True), (2, False)])
def test_paged_attention_equals_contiguous(oracle_mod, bits, hybrid):
    O = oracle_mod
    rng = np.random.default_rng(7 * bits)
    fmt = O.Format(bits, 128, hybrid)
    B, Hq, Hkv, n_packed, n_res, cap = 2, 8, 2, 384, 20, 32
    rows = B * Hkv
    ksrc = _f16(rng.standard_normal((rows, n_packed, 128)))
    vsrc = _f16(rng.standard_normal((rows, n_packed, 128)))
    kp = O.quantize_pack(fmt, ksrc)
    vp = O.quantize_pack(fmt, vsrc)
    kres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    ref = O.attention(fmt, q, Hkv, kp, vp, n_packed, kres, vres, n_res, sm=SM)
    nb = n_packed // 128
    tbl, npool = P.make_table(rng, B, [nb] * B, n_pool_blocks=2 * B * nb)
    bb = fmt.block_bytes
    kpool = P.new_pool(npool, Hkv, bb, fill=0xFF)          # unused blocks hold NaN patterns
    vpool = P.new_pool(npool, Hkv, bb, fill=0xFF)
    for b in range(B):
        for h in range(Hkv):
            for j in range(nb):
                kpool[tbl[b, j], h] = kp[b * Hkv + h, j * bb:(j + 1) * bb]
                vpool[tbl[b, j], h] = vp[b * Hkv + h, j * bb:(j + 1) * bb]
    state = np.array([[n_packed, n_res, 0, 0]] * B, np.int32)
    got = O.attention_paged(fmt, q, Hkv, kpool, vpool, tbl, state, kres, vres, sm=SM)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_ragged_packed_tail_equals_the_same_values_in_the_window(oracle_mod, bits):
    O = oracle_mod
    rng = np.random.default_rng(100 + bits)
    fmt = O.Format(bits, 128, False)
    B, Hq, Hkv = 3, 8, 2
    n_packed = [300, 5, 128]
    n_res = [10, 0, 3]
    cap = 16
    T = max(n_packed)
    src_k = _grid_tokens(rng, B * Hkv, T, bits)
    src_v = _grid_tokens(rng, B * Hkv, T, bits)
    tbl, npool = P.make_table(rng, B, [P.blocks_for(n) for n in n_packed], n_pool_blocks=9)
    kpool = P.new_pool(npool, Hkv, fmt.block_bytes, fill=0xFF)
    vpool = P.new_pool(npool, Hkv, fmt.block_bytes, fill=0xFF)
    O.pack_tokens_paged(fmt, src_k, B, Hkv, n_packed, [0] * B, kpool, tbl)
    O.pack_tokens_paged(fmt, src_v, B, Hkv, n_packed, [0] * B, vpool, tbl)
    kres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    state = np.array([[n_packed[b], n_res[b], 0, 0] for b in range(B)], np.int32)
    got = O.attention_paged(fmt, q, Hkv, kpool, vpool, tbl, state, kres, vres, sm=SM)
    for b in range(B):
        # same sequence with whole blocks packed contiguously and the tail in the window
        whole = n_packed[b] // 128 * 128
        tail = n_packed[b] - whole
        kw = np.zeros((1, Hkv, tail + cap, 128), np.float16)
        vw = np.zeros_like(kw)
        kw[0, :, :tail] = src_k[b * Hkv:(b + 1) * Hkv, whole:n_packed[b]]
        vw[0, :, :tail] = src_v[b * Hkv:(b + 1) * Hkv, whole:n_packed[b]]
        kw[0, :, tail:] = kres[b]
        vw[0, :, tail:] = vres[b]
        if whole:
            kp = O.quantize_pack(fmt, np.ascontiguousarray(src_k[b * Hkv:(b + 1) * Hkv, :whole]))
            vp = O.quantize_pack(fmt, np.ascontiguousarray(src_v[b * Hkv:(b + 1) * Hkv, :whole]))
        else:
            kp = vp = np.zeros((Hkv, 0), np.uint8)
        ref = O.attention(fmt, q[b:b + 1], Hkv, kp, vp, whole, kw, vw, tail + n_res[b], sm=SM)
        assert np.array_equal(got[b], ref[0])


def test_split_ranges_tile_the_sequence(oracle_mod):
    O = oracle_mod
    for n_packed in (0, 1, 31, 32, 33, 300, 4096, 5000):
        for n_res in (0, 1, 128):
            for S in (1, 2, 3, 7, 64):
                if n_packed + n_res == 0:
                    continue
                cover = []
                for s in range(S):
                    lo, hi = O.paged_split_range(n_packed, n_res, S, s)
                    assert 0 <= lo <= hi <= n_packed + n_res
                    if hi > lo:
                        assert lo % 32 == 0 or lo == n_packed
                        cover.append((lo, hi))
                flat = [t for lo, hi in cover for t in range(lo, hi)]
                assert flat == list(range(n_packed + n_res)), (n_packed, n_res, S)
                if S > 1 and n_res:
                    assert O.paged_split_range(n_packed, n_res, S, S - 1) == (n_packed,
                                                                              n_packed + n_res)


@pytest.mark.parametrize("S", [1, 3, 6])
def test_paged_split_partials_merge_to_one_pass(oracle_mod, S):
    O = oracle_mod
    rng = np.random.default_rng(S)
    fmt = O.Format(4, 128, False)
    B, Hq, Hkv, cap = 3, 4, 1, 8
    n_packed, n_res = [77, 0, 260], [8, 3, 0]
    tbl, npool = P.make_table(rng, B, [P.blocks_for(n) for n in n_packed])
    kpool = P.new_pool(npool, Hkv, fmt.block_bytes, fill=0)
    vpool = P.new_pool(npool, Hkv, fmt.block_bytes, fill=0)
    src = _f16(rng.standard_normal((B * Hkv, 260, 128)))
    O.pack_tokens_paged(fmt, src, B, Hkv, n_packed, [0] * B, kpool, tbl)
    O.pack_tokens_paged(fmt, src[:, ::-1].copy(), B, Hkv, n_packed, [0] * B, vpool, tbl)
    kres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)) * 2)
    state = np.array([[n_packed[b], n_res[b], 0, 0] for b in range(B)], np.int32)
    one = O.attention_paged(fmt, q, Hkv, kpool, vpool, tbl, state, kres, vres, sm=SM)
    po, pl = O.attention_paged(fmt, q, Hkv, kpool, vpool, tbl, state, kres, vres, sm=SM, S=S)
    for b in range(B):
        for s in range(S):
            lo, hi = O.paged_split_range(n_packed[b], n_res[b], S, s)
            assert np.isneginf(pl[b, :, s]).all() == (hi == lo)
    assert np.max(np.abs(O.combine(po, pl) - one)) < 1e-12
