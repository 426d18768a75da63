"""GPU parity of the paged cache path (kvq_pack_tokens_paged, kvq_append_evict,
kvq_decode_attention_paged) against the CPU oracle.

Bars: pool bytes, windows and sequence states bit-exact; decode partials and the combined
output within the attention bar of the other decode tests (max-abs 2e-3, rel-L2 1e-3)
against the fp64 oracle; and, where the paged cache holds exactly a contiguous cache,
partials bit-identical to kvq_decode_attention's. Pools start filled with 0xFF bytes (fp16
NaN scale/zero patterns) so that reading past a sequence's length shows up."""
import numpy as np
import pytest
import torch

import paged_common as P
import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _layout(kind, npool, Hkv, bb):
    """(numpy pool shape, block_stride, head_stride) of a pool layout."""
    if kind == "block_major":                  # [blocks][Hkv][bb]
        return (npool, Hkv, bb), Hkv * bb, bb
    return (Hkv, npool, bb), bb, npool * bb    # [Hkv][blocks][bb]


def _dev(a):
    from gpu_common import dev
    return dev(a)


@pytest.mark.parametrize("layout", ["block_major", "head_major"])
@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, True), (2, False), (2, True)])
def test_pack_tokens_paged_bytes(oracle_mod, layout, bits, hybrid):
    O = oracle_mod
    rng = np.random.default_rng(bits * 3 + hybrid)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    B, Hkv = 4, 3
    count = np.array([300, 0, 1, 129], np.int32)
    start = np.array([0, 5, 127, 77], np.int32)
    T = int(count.max())
    nblocks = [P.blocks_for(s + c) if c else 1 for s, c in zip(start, count)]
    tbl, npool = P.make_table(rng, B, nblocks, n_pool_blocks=sum(nblocks) + 3)
    shape, bs, hs = _layout(layout, npool, Hkv, fmt.block_bytes)
    src = _f16(rng.standard_normal((B * Hkv, T + 3, 128)) *
               rng.uniform(0.05, 8, (B * Hkv, 1, 128)))
    print(f"[pack_paged] bits={bits} hybrid={hybrid} layout={layout}", flush=True)
    ref = np.full(shape, 0xFF, np.uint8)
    O.pack_tokens_paged(ofmt, src[:, :T], B, Hkv, count, start, ref, tbl, block_stride=bs,
                        head_stride=hs)
    pool = _dev(np.full(shape, 0xFF, np.uint8))
    srcd = _dev(src)
    K.kvq_pack_tokens_paged(fmt, srcd, B, Hkv, (T + 3) * 128, 128, _dev(count), _dev(start), T,
                            pool, npool, bs, hs, _dev(tbl), tbl.shape[1])
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref)


def test_pack_tokens_paged_skips_unmapped_blocks(oracle_mod):
    """A table entry of -1 or past the pool: nothing is written for those tokens."""
    O = oracle_mod
    rng = np.random.default_rng(3)
    fmt, ofmt = K.Format(4), O.Format(4)
    B, Hkv = 3, 2
    count = np.array([200, 100, 50], np.int32)
    start = np.zeros(3, np.int32)
    tbl, npool = P.make_table(rng, B, [2, 1, 1])
    bad = tbl.copy()
    bad[1, 0] = -1
    bad[2, 0] = npool + 5
    shape, bs, hs = _layout("block_major", npool, Hkv, fmt.block_bytes)
    src = _f16(rng.standard_normal((B * Hkv, 200, 128)))
    ref = np.full(shape, 0xFF, np.uint8)
    O.pack_tokens_paged(ofmt, src, B, Hkv, [200, 0, 0], start, ref, tbl, block_stride=bs,
                        head_stride=hs)
    pool = _dev(np.full(shape, 0xFF, np.uint8))
    K.kvq_pack_tokens_paged(fmt, _dev(src), B, Hkv, 200 * 128, 128, _dev(count), _dev(start), 200,
                            pool, npool, bs, hs, _dev(bad), bad.shape[1])
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref)


def _state(rows):
    return np.ascontiguousarray(np.array(rows, np.int32).reshape(-1, 4))


@pytest.mark.parametrize("bits,hybrid,cap,n_sink,steps", [
    (4, False, 16, 4, 200),
    (2, True, 8, 0, 150),
    (3, False, 128, 32, 300),
])
def test_append_evict_matches_oracle(oracle_mod, bits, hybrid, cap, n_sink, steps):
    O = oracle_mod
    rng = np.random.default_rng(cap + bits)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    B, Hkv = 3, 4
    # sequences: empty window; full window with some packed tokens; partly filled window
    st0 = _state([[0, 0, n_sink, 0], [77, cap, n_sink + (5 % (cap - n_sink)), 0],
                  [130, min(3, cap - 1), n_sink, 0]])
    max_packed = int(st0[:, 0].max()) + steps + 1
    tbl, npool = P.make_table(rng, B, [P.blocks_for(max_packed)] * B)
    shape, bs, hs = _layout("block_major", npool, Hkv, fmt.block_bytes)
    kpool = rng.integers(0, 256, shape, dtype=np.uint8)       # earlier tokens' bytes
    vpool = rng.integers(0, 256, shape, dtype=np.uint8)
    kres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    vres = _f16(rng.standard_normal((B, Hkv, cap, 128)))
    new_k = _f16(rng.standard_normal((steps, B, Hkv, 128)) * rng.uniform(0.1, 5, (1, 1, Hkv, 128)))
    new_v = _f16(rng.standard_normal((steps, B, Hkv, 128)))
    dk, dv, dkr, dvr, dst = (_dev(kpool), _dev(vpool), _dev(kres), _dev(vres), _dev(st0))
    dtbl = _dev(tbl)
    okp, ovp, okr, ovr, ost = kpool.copy(), vpool.copy(), kres.copy(), vres.copy(), st0.copy()
    print(f"[append_evict] bits={bits} hybrid={hybrid} cap={cap} sink={n_sink} steps={steps}",
          flush=True)
    dnk, dnv = _dev(new_k), _dev(new_v)
    for i in range(steps):
        K.kvq_append_evict(fmt, dnk[i], dnv[i], dkr, dvr, cap, n_sink, dk, dv, npool, bs, hs,
                           dtbl, tbl.shape[1], dst, B, Hkv)
        O.append_evict(ofmt, new_k[i], new_v[i], okr, ovr, n_sink, okp, ovp, tbl, ost,
                       block_stride=bs, head_stride=hs)
        if i in (steps // 3, steps - 1):
            torch.cuda.synchronize()
            assert np.array_equal(dst.cpu().numpy(), ost), f"state after step {i}"
            assert np.array_equal(dkr.cpu().numpy().view(np.uint16), okr.view(np.uint16))
            assert np.array_equal(dvr.cpu().numpy().view(np.uint16), ovr.view(np.uint16))
            assert np.array_equal(dk.cpu().numpy(), okp), f"K pool after step {i}"
            assert np.array_equal(dv.cpu().numpy(), ovp), f"V pool after step {i}"


def _paged_case(O, rng, fmt, ofmt, B, Hq, Hkv, n_packed, n_res, cap, layout="block_major",
                scale=1.0):
    """A paged cache built by the oracle (pool bytes, table, state, windows) and q."""
    T = max(max(n_packed), 1)
    tbl, npool = P.make_table(rng, B, [max(P.blocks_for(n), 1) for n in n_packed],
                              n_pool_blocks=sum(max(P.blocks_for(n), 1) for n in n_packed) + 2)
    shape, bs, hs = _layout(layout, npool, Hkv, fmt.block_bytes)
    kpool = np.full(shape, 0xFF, np.uint8)
    vpool = np.full(shape, 0xFF, np.uint8)
    ks = _f16(rng.standard_normal((B * Hkv, T, 128)) * scale)
    vs = _f16(rng.standard_normal((B * Hkv, T, 128)) * scale)
    zero = np.zeros(B, np.int32)
    O.pack_tokens_paged(ofmt, ks, B, Hkv, n_packed, zero, kpool, tbl, block_stride=bs,
                        head_stride=hs)
    O.pack_tokens_paged(ofmt, vs, B, Hkv, n_packed, zero, vpool, tbl, block_stride=bs,
                        head_stride=hs)
    kres = _f16(rng.standard_normal((B, Hkv, cap, 128)) * scale)
    vres = _f16(rng.standard_normal((B, Hkv, cap, 128)) * scale)
    state = _state([[n_packed[b], n_res[b], 0, 0] for b in range(B)])
    q = _f16(rng.standard_normal((B, Hq, 128)))
    return dict(tbl=tbl, npool=npool, bs=bs, hs=hs, kpool=kpool, vpool=vpool, kres=kres,
                vres=vres, state=state, q=q, cap=cap)


def _gpu_paged_decode(fmt, c, B, Hq, Hkv, S_):
    from gpu_common import DEV
    po = torch.full((B, Hq, S_, 128), float("nan"), dtype=torch.float32, device=DEV)
    pl = torch.full((B, Hq, S_), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_paged(fmt, _dev(c["q"]), B, Hq, Hkv, _dev(c["kpool"]), _dev(c["vpool"]),
                                 c["npool"], c["bs"], c["hs"], _dev(c["tbl"]), c["tbl"].shape[1],
                                 _dev(c["state"]), _dev(c["kres"]), _dev(c["vres"]), c["cap"], SM,
                                 S_, po, pl)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F32)
    torch.cuda.synchronize()
    return out.cpu().numpy(), po.cpu().numpy(), pl.cpu().numpy()


DECODE_CASES = [
    # bits, hybrid, B, Hq, Hkv, n_packed per sequence, n_res per sequence, cap, S, layout
    (4, False, 4, 8, 2, [300, 1, 31, 1000], [10, 0, 128, 5], 128, 3, "block_major"),
    (4, False, 3, 32, 8, [33, 4096, 0], [0, 17, 40], 64, 5, "head_major"),
    (3, True, 2, 6, 1, [517, 64], [3, 3], 16, 2, "block_major"),
    (2, False, 5, 16, 16, [1, 2, 127, 128, 129], [1, 0, 0, 7, 2], 8, 1, "block_major"),
    (2, True, 2, 12, 1, [2000, 95], [0, 1], 4, 7, "head_major"),
    (4, False, 2, 20, 2, [640, 333], [16, 16], 16, 4, "block_major"),   # 10 heads: chunks 4+4+2
    (4, False, 2, 8, 2, [32768, 700], [128, 3], 128, 1024, "head_major"),  # the split limit
]


@pytest.mark.parametrize("bits,hybrid,B,Hq,Hkv,n_packed,n_res,cap,S_,layout", DECODE_CASES)
def test_paged_decode_matches_oracle(oracle_mod, bits, hybrid, B, Hq, Hkv, n_packed, n_res, cap,
                                     S_, layout):
    from gpu_common import assert_close
    O = oracle_mod
    rng = np.random.default_rng(sum(n_packed) + bits)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    c = _paged_case(O, rng, fmt, ofmt, B, Hq, Hkv, n_packed, n_res, cap, layout)
    print(f"[decode_paged] bits={bits} hybrid={hybrid} B={B} Hq={Hq} Hkv={Hkv} "
          f"n_packed={n_packed} n_res={n_res} S={S_} {layout}", flush=True)
    out, po, pl = _gpu_paged_decode(fmt, c, B, Hq, Hkv, S_)
    rpo, rpl = O.attention_paged(ofmt, c["q"], Hkv, c["kpool"], c["vpool"], c["tbl"], c["state"],
                                 c["kres"], c["vres"], sm=SM, S=S_, block_stride=c["bs"],
                                 head_stride=c["hs"])
    empty = np.isneginf(rpl)
    assert np.array_equal(np.isneginf(pl), empty), "empty splits differ"
    assert np.all(po[empty] == 0)
    assert np.max(np.abs(pl[~empty] - rpl[~empty])) < 1e-3
    assert_close(po[~empty], rpo[~empty], "partials")
    ref = O.attention_paged(ofmt, c["q"], Hkv, c["kpool"], c["vpool"], c["tbl"], c["state"],
                            c["kres"], c["vres"], sm=SM, block_stride=c["bs"], head_stride=c["hs"])
    assert_close(out, ref, "attention")


def test_paged_decode_equals_contiguous_decode():
    """The pages hold a contiguous cache's blocks, scattered over the pool (uniform lengths,
    whole blocks): the paged kernel's partials equal kvq_decode_attention's up to fp32
    rounding (the two kernels are compiled separately, so the compiler may fuse a product
    and a sum in one and not in the other)."""
    from gpu_common import DEV, gpu_quantize
    rng = np.random.default_rng(21)
    fmt = K.Format(4)
    B, Hq, Hkv, n_packed, n_res, S_ = 2, 16, 4, 1024, 50, 5
    rows, nb, bb = B * Hkv, n_packed // 128, fmt.block_bytes
    ks = _f16(rng.standard_normal((rows, n_packed, 128)))
    vs = _f16(rng.standard_normal((rows, n_packed, 128)))
    kp, vp = gpu_quantize(fmt, ks), gpu_quantize(fmt, vs)
    kr = _dev(_f16(rng.standard_normal((B, Hkv, 128, 128))))
    vr = _dev(_f16(rng.standard_normal((B, Hkv, 128, 128))))
    q = _dev(_f16(rng.standard_normal((B, Hq, 128))))
    tbl, npool = P.make_table(rng, B, [nb] * B, n_pool_blocks=B * nb + 3)
    # pool [blocks][Hkv][bb]: block tbl[b][e] holds block e of rows b*Hkv .. b*Hkv+Hkv-1
    idx = torch.from_numpy(tbl.reshape(-1).astype(np.int64)).to(DEV)
    kpool = torch.full((npool, Hkv, bb), 0xFF, dtype=torch.uint8, device=DEV)
    vpool = torch.full_like(kpool, 0xFF)
    kpool[idx] = kp.view(B, Hkv, nb, bb).permute(0, 2, 1, 3).reshape(B * nb, Hkv, bb)
    vpool[idx] = vp.view(B, Hkv, nb, bb).permute(0, 2, 1, 3).reshape(B * nb, Hkv, bb)
    state = _state([[n_packed, n_res, 0, 0]] * B)
    po1 = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl1 = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    po2, pl2 = torch.empty_like(po1), torch.empty_like(pl1)
    K.kvq_decode_attention(fmt, q, B, Hq, Hkv, kp, vp, nb * bb, n_packed, kr, vr, 128, n_res, SM,
                           S_, po1, pl1)
    K.kvq_decode_attention_paged(fmt, q, B, Hq, Hkv, kpool, vpool, npool, Hkv * bb, bb,
                                 _dev(tbl), nb, _dev(state), kr, vr, 128, SM, S_, po2, pl2)
    torch.cuda.synchronize()
    do = (po1 - po2).abs().max().item()
    dl = (pl1 - pl2).abs().max().item()
    print(f"[paged vs contiguous] max |d part_o| = {do:.3e}, max |d lse| = {dl:.3e}", flush=True)
    assert do <= 1e-5 and dl <= 1e-5


def test_prefill_then_sliding_steps_then_decode(oracle_mod):
    """A serving-shaped run: ragged prompts packed with kvq_pack_tokens_paged (sinks and
    recent tokens placed in the windows), 140 steps of kvq_append_evict, then the decode --
    all on the GPU -- against the oracle doing the same."""
    from gpu_common import DEV, assert_close
    O = oracle_mod
    rng = np.random.default_rng(99)
    fmt, ofmt = K.Format(4), O.Format(4)
    B, Hq, Hkv, cap, n_sink, steps, S_ = 3, 8, 2, 32, 4, 140, 4
    prompt = [500, 20, 1300]
    max_tokens = max(prompt) + steps
    tbl, npool = P.make_table(rng, B, [P.blocks_for(max_tokens)] * B)
    shape, bs, hs = _layout("block_major", npool, Hkv, fmt.block_bytes)
    toks_k = _f16(rng.standard_normal((B * Hkv, max(prompt), 128)))
    toks_v = _f16(rng.standard_normal((B * Hkv, max(prompt), 128)))
    # window: sinks + most recent prompt tokens; packed: the rest, in order
    kres = np.zeros((B, Hkv, cap, 128), np.float16)
    vres = np.zeros_like(kres)
    count, start = np.zeros(B, np.int32), np.zeros(B, np.int32)
    mid_k = np.zeros((B * Hkv, max(prompt), 128), np.float16)
    mid_v = np.zeros_like(mid_k)
    state = np.zeros((B, 4), np.int32)
    for b, n in enumerate(prompt):
        r = slice(b * Hkv, (b + 1) * Hkv)
        if n <= cap:
            kres[b, :, :n] = toks_k[r, :n]
            vres[b, :, :n] = toks_v[r, :n]
            state[b] = [0, n, n_sink, 0]
            continue
        recent = cap - n_sink
        kres[b, :, :n_sink] = toks_k[r, :n_sink]
        vres[b, :, :n_sink] = toks_v[r, :n_sink]
        kres[b, :, n_sink:] = toks_k[r, n - recent:n]
        vres[b, :, n_sink:] = toks_v[r, n - recent:n]
        m = n - cap
        mid_k[r, :m] = toks_k[r, n_sink:n_sink + m]
        mid_v[r, :m] = toks_v[r, n_sink:n_sink + m]
        count[b] = m
        state[b] = [m, cap, n_sink, 0]
    T = max(prompt)
    okp = np.full(shape, 0xFF, np.uint8)
    ovp = np.full(shape, 0xFF, np.uint8)
    O.pack_tokens_paged(ofmt, mid_k, B, Hkv, count, start, okp, tbl, block_stride=bs, head_stride=hs)
    O.pack_tokens_paged(ofmt, mid_v, B, Hkv, count, start, ovp, tbl, block_stride=bs, head_stride=hs)
    dk, dv = _dev(np.full(shape, 0xFF, np.uint8)), _dev(np.full(shape, 0xFF, np.uint8))
    dtbl, dcount, dstart = _dev(tbl), _dev(count), _dev(start)
    K.kvq_pack_tokens_paged(fmt, _dev(mid_k), B, Hkv, T * 128, 128, dcount, dstart, T, dk, npool,
                            bs, hs, dtbl, tbl.shape[1])
    K.kvq_pack_tokens_paged(fmt, _dev(mid_v), B, Hkv, T * 128, 128, dcount, dstart, T, dv, npool,
                            bs, hs, dtbl, tbl.shape[1])
    dkr, dvr, dst = _dev(kres), _dev(vres), _dev(state)
    okr, ovr, ost = kres.copy(), vres.copy(), state.copy()
    new_k = _f16(rng.standard_normal((steps, B, Hkv, 128)))
    new_v = _f16(rng.standard_normal((steps, B, Hkv, 128)))
    dnk, dnv = _dev(new_k), _dev(new_v)
    print("[serving run] prefill packed; steps", flush=True)
    for i in range(steps):
        K.kvq_append_evict(fmt, dnk[i], dnv[i], dkr, dvr, cap, n_sink, dk, dv, npool, bs, hs, dtbl,
                           tbl.shape[1], dst, B, Hkv)
        O.append_evict(ofmt, new_k[i], new_v[i], okr, ovr, n_sink, okp, ovp, tbl, ost,
                       block_stride=bs, head_stride=hs)
    q = _f16(rng.standard_normal((B, Hq, 128)))
    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_paged(fmt, _dev(q), B, Hq, Hkv, dk, dv, npool, bs, hs, dtbl,
                                 tbl.shape[1], dst, dkr, dvr, cap, SM, S_, po, pl)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), ost)
    assert np.array_equal(dk.cpu().numpy(), okp) and np.array_equal(dv.cpu().numpy(), ovp)
    ref = O.attention_paged(ofmt, q, Hkv, okp, ovp, tbl, ost, okr, ovr, sm=SM, block_stride=bs,
                            head_stride=hs)
    assert_close(out.cpu().numpy(), ref, "serving run attention")


@pytest.mark.slow
def test_paged_decode_full_size_ragged(oracle_mod):
    """16 sequences of 1K..32K tokens, Llama-8B heads (32 q / 8 kv), 4-bit, the split count
    the library suggests for ragged batches: every output against the oracle."""
    from gpu_common import assert_close
    O = oracle_mod
    wl = S.PAGED_WORKLOADS["paged_ragged_b16"]
    x = S.make_paged_inputs(wl)
    fmt, ofmt = K.Format(wl.bits), O.Format(wl.bits)
    print(f"[decode_paged] full size {wl.name}", flush=True)
    c = _paged_from_inputs(O, ofmt, wl, x)
    S_ = K.suggest_splits_paged(int(x.n_packed.sum()), int(x.n_packed.max()), wl.Hkv, 256)
    out, po, pl = _gpu_paged_decode(fmt, c, wl.B, wl.Hq, wl.Hkv, S_)
    ref = O.attention_paged(ofmt, c["q"], wl.Hkv, c["kpool"], c["vpool"], c["tbl"], c["state"],
                            c["kres"], c["vres"], sm=SM, block_stride=c["bs"], head_stride=c["hs"])
    assert_close(out, ref, "full-size paged attention")


def _paged_from_inputs(O, ofmt, wl, x):
    shape = (x.n_pool_blocks, wl.Hkv, ofmt.block_bytes)
    kpool = np.zeros(shape, np.uint8)
    vpool = np.zeros(shape, np.uint8)
    for b in range(wl.B):
        n = int(x.n_packed[b])
        if n:
            O.pack_tokens_paged(ofmt, x.k_src[b], 1, wl.Hkv, [n], [0], kpool, x.table[b:b + 1])
            O.pack_tokens_paged(ofmt, x.v_src[b], 1, wl.Hkv, [n], [0], vpool, x.table[b:b + 1])
    state = _state([[x.n_packed[b], x.n_res[b], 0, 0] for b in range(wl.B)])
    return dict(tbl=x.table, npool=x.n_pool_blocks, bs=wl.Hkv * ofmt.block_bytes,
                hs=ofmt.block_bytes, kpool=kpool, vpool=vpool, kres=x.k_res, vres=x.v_res,
                state=state, q=x.q, cap=x.k_res.shape[2])


def test_paged_decode_with_key_norm_equals_scaled_q(oracle_mod):
    """A paged cache of key-normalized keys: passing the factors to the paged decode gives
    the partials of the paged decode on q multiplied by them with kvq_channel_scale."""
    from gpu_common import DEV
    O = oracle_mod
    rng = np.random.default_rng(77)
    fmt, ofmt = K.Format(4), O.Format(4)
    B, Hq, Hkv, S_ = 3, 16, 4, 3
    c = _paged_case(O, rng, fmt, ofmt, B, Hq, Hkv, [700, 33, 0], [10, 0, 64], 64)
    norm = (2.0 ** rng.uniform(-3, 3, (B * Hkv, 128))).astype(np.float32)
    nd, qd = _dev(norm), _dev(c["q"])
    qs = torch.empty_like(qd)
    K.kvq_channel_scale(qd, B * Hq, 1, 128, 128, 128, nd, Hq // Hkv, K.KVQ_SCALE_MULTIPLY, qs,
                        128, 128)
    args = (B, Hq, Hkv, _dev(c["kpool"]), _dev(c["vpool"]), c["npool"], c["bs"], c["hs"],
            _dev(c["tbl"]), c["tbl"].shape[1], _dev(c["state"]), _dev(c["kres"]),
            _dev(c["vres"]), c["cap"], SM, S_)
    outs = []
    for q, kn in ((qd, nd), (qs, None)):
        po = torch.full((B, Hq, S_, 128), float("nan"), dtype=torch.float32, device=DEV)
        pl = torch.full((B, Hq, S_), float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_decode_attention_paged(fmt, q, *args, po, pl, key_norm=kn)
        outs.append((po, pl))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_serving_run_with_key_normalization(oracle_mod):
    """Everything together: per-sequence key-channel factors from the prompt keys, prompt
    keys divided by them and packed into the pages, 60 steps whose new keys are divided
    before they enter the window (kvq_channel_scale into a staging buffer, then
    kvq_append_evict), and the paged decode with the factors -- all on the GPU -- against
    the oracle doing the same steps."""
    from gpu_common import DEV, assert_close
    O = oracle_mod
    rng = np.random.default_rng(123)
    fmt, ofmt = K.Format(3), O.Format(3)
    B, Hq, Hkv, cap, n_sink, steps, S_ = 2, 8, 2, 16, 2, 60, 3
    prompt = [400, 150]
    rows = B * Hkv
    T = max(prompt)
    ch_mult = np.ones(128, np.float32)
    ch_mult[[5, 90]] = 9.0                                       # outlier key channels
    toks_k = _f16(rng.standard_normal((rows, T, 128)) * ch_mult)
    toks_v = _f16(rng.standard_normal((rows, T, 128)))
    new_k = _f16(rng.standard_normal((steps, B, Hkv, 128)) * ch_mult)
    new_v = _f16(rng.standard_normal((steps, B, Hkv, 128)))
    q = _f16(rng.standard_normal((B, Hq, 128)))
    tbl, npool = P.make_table(rng, B, [P.blocks_for(p + steps) for p in prompt])
    shape, bs, hs = _layout("block_major", npool, Hkv, fmt.block_bytes)
    # prompt split: sinks + recent in the window, the middle packed (per sequence)
    count = np.zeros(B, np.int32)
    state = np.zeros((B, 4), np.int32)
    mid_idx = []
    for b, n in enumerate(prompt):
        m = n - cap
        count[b] = m
        state[b] = [m, cap, n_sink, 0]
        mid_idx.append(np.arange(n_sink, n_sink + m))
    # ---- oracle
    norm = np.zeros((rows, 128), np.float32)
    for b, n in enumerate(prompt):                    # factors over each sequence's prompt
        norm[b * Hkv:(b + 1) * Hkv] = O.key_norm(toks_k[b * Hkv:(b + 1) * Hkv, :n])
    kn_all = O.channel_scale(toks_k, norm).view(np.float16)
    mid_k = np.zeros((rows, T, 128), np.float16)
    mid_v = np.zeros_like(mid_k)
    kres = np.zeros((B, Hkv, cap, 128), np.float16)
    vres = np.zeros_like(kres)
    for b, n in enumerate(prompt):
        r = slice(b * Hkv, (b + 1) * Hkv)
        mid_k[r, :count[b]] = kn_all[r][:, mid_idx[b]]
        mid_v[r, :count[b]] = toks_v[r][:, mid_idx[b]]
        kres[b, :, :n_sink] = kn_all[r, :n_sink]
        vres[b, :, :n_sink] = toks_v[r, :n_sink]
        kres[b, :, n_sink:] = kn_all[r, n - (cap - n_sink):n]
        vres[b, :, n_sink:] = toks_v[r, n - (cap - n_sink):n]
    okp = np.full(shape, 0xFF, np.uint8)
    ovp = np.full(shape, 0xFF, np.uint8)
    zero = np.zeros(B, np.int32)
    O.pack_tokens_paged(ofmt, mid_k, B, Hkv, count, zero, okp, tbl)
    O.pack_tokens_paged(ofmt, mid_v, B, Hkv, count, zero, ovp, tbl)
    okr, ovr, ost = kres.copy(), vres.copy(), state.copy()
    for i in range(steps):
        kn = O.channel_scale(new_k[i].reshape(rows, 1, 128), norm).view(np.float16).reshape(B, Hkv, 128)
        O.append_evict(ofmt, kn, new_v[i], okr, ovr, n_sink, okp, ovp, tbl, ost)
    qn = O.channel_scale(q.reshape(B * Hq, 1, 128), norm, rows_per_norm=Hq // Hkv,
                         multiply=True).view(np.float16).reshape(B, Hq, 128)
    ref = O.attention_paged(ofmt, qn, Hkv, okp, ovp, tbl, ost, okr, ovr, sm=SM)

    # ---- GPU
    print("[serving+knorm] prefill", flush=True)
    dk_all = _dev(toks_k)
    dnorm = torch.empty((rows, 128), dtype=torch.float32, device=DEV)
    for b, n in enumerate(prompt):
        K.kvq_key_norm(dk_all[b * Hkv:(b + 1) * Hkv], Hkv, n, T * 128, 128, 128,
                       dnorm[b * Hkv:(b + 1) * Hkv])
    K.kvq_channel_scale(dk_all, rows, T, T * 128, 128, 128, dnorm, 1, K.KVQ_SCALE_DIVIDE, dk_all,
                        T * 128, 128)
    torch.cuda.synchronize()
    assert np.array_equal(dnorm.cpu().numpy().view(np.uint32), norm.view(np.uint32))
    assert np.array_equal(dk_all.cpu().numpy().view(np.uint16), kn_all.view(np.uint16))
    # the same split of the prompt, gathered on the GPU from the normalized keys
    dmid_k = torch.zeros((rows, T, 128), dtype=torch.float16, device=DEV)
    dmid_v = torch.zeros_like(dmid_k)
    dv_all = _dev(toks_v)
    dkres = torch.zeros((B, Hkv, cap, 128), dtype=torch.float16, device=DEV)
    dvres = torch.zeros_like(dkres)
    for b, n in enumerate(prompt):
        r = slice(b * Hkv, (b + 1) * Hkv)
        idx = torch.from_numpy(mid_idx[b]).to(DEV)
        dmid_k[r, :count[b]] = dk_all[r][:, idx]
        dmid_v[r, :count[b]] = dv_all[r][:, idx]
        dkres[b, :, :n_sink] = dk_all[r, :n_sink]
        dvres[b, :, :n_sink] = dv_all[r, :n_sink]
        dkres[b, :, n_sink:] = dk_all[r, n - (cap - n_sink):n]
        dvres[b, :, n_sink:] = dv_all[r, n - (cap - n_sink):n]
    dk, dv = _dev(np.full(shape, 0xFF, np.uint8)), _dev(np.full(shape, 0xFF, np.uint8))
    dtbl, dcount, dzero = _dev(tbl), _dev(count), _dev(zero)
    K.kvq_pack_tokens_paged(fmt, dmid_k, B, Hkv, T * 128, 128, dcount, dzero, T, dk, npool, bs, hs,
                            dtbl, tbl.shape[1])
    K.kvq_pack_tokens_paged(fmt, dmid_v, B, Hkv, T * 128, 128, dcount, dzero, T, dv, npool, bs, hs,
                            dtbl, tbl.shape[1])
    dkr, dvr, dst = dkres, dvres, _dev(state)
    dnk, dnv = _dev(new_k), _dev(new_v)
    stage = torch.empty((B, Hkv, 128), dtype=torch.float16, device=DEV)
    print("[serving+knorm] steps", flush=True)
    for i in range(steps):
        K.kvq_channel_scale(dnk[i], rows, 1, 128, 128, 128, dnorm, 1, K.KVQ_SCALE_DIVIDE, stage,
                            128, 128)
        K.kvq_append_evict(fmt, stage, dnv[i], dkr, dvr, cap, n_sink, dk, dv, npool, bs, hs, dtbl,
                           tbl.shape[1], dst, B, Hkv)
    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    K.kvq_decode_attention_paged(fmt, _dev(q), B, Hq, Hkv, dk, dv, npool, bs, hs, dtbl,
                                 tbl.shape[1], dst, dkr, dvr, cap, SM, S_, po, pl, key_norm=dnorm)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), ost)
    assert np.array_equal(dk.cpu().numpy(), okp) and np.array_equal(dv.cpu().numpy(), ovp)
    assert np.array_equal(dkr.cpu().numpy().view(np.uint16), okr.view(np.uint16))
    assert_close(out.cpu().numpy(), ref, "serving run with key normalization")


@pytest.mark.parametrize("bits,hybrid,Hq,Hkv,cap,n_sink,steps,S_,layout,knorm", [
    (4, False, 8, 2, 16, 4, 40, 3, "block_major", False),  # gq 4: the update inside the decode
    (4, False, 32, 8, 8, 0, 30, 16, "head_major", False),
    (2, True, 4, 4, 8, 2, 30, 2, "block_major", False),    # gq 1
    (3, False, 6, 2, 16, 3, 25, 1, "block_major", False),  # gq 3, one split
    (3, True, 16, 2, 8, 1, 20, 4, "head_major", False),    # gq 8: two launches inside the call
    (4, False, 8, 2, 16, 4, 12, 3, "block_major", True),   # with key-channel factors
    (2, True, 16, 2, 8, 0, 12, 2, "head_major", True),     # the same through two launches
    (2, False, 8, 2, 16, 4, 40, 5, "block_major", False),  # 2-bit asym, gq 4 (transposed K in LDS)
    (3, False, 8, 2, 16, 4, 40, 7, "block_major", False),  # 3-bit, gq 4
])
def test_paged_append_equals_update_then_decode(oracle_mod, bits, hybrid, Hq, Hkv, cap, n_sink,
                                                steps, S_, layout, knorm):
    """kvq_decode_attention_paged_append equals kvq_append_evict followed by
    kvq_decode_attention_paged, step after step: windows, pools, states and partials bit
    for bit (sequences that start with an empty window, a full one, a partly filled one, and
    packed lengths that put the evicted token at every position of a tile and of a block);
    the final output also against the oracle."""
    from gpu_common import DEV, assert_close
    O = oracle_mod
    rng = np.random.default_rng(bits * 100 + Hq + cap)
    fmt, ofmt = K.Format(bits, 128, hybrid), O.Format(bits, 128, hybrid)
    B = 4
    n_packed = [0, 77, 127, 31]
    n_res = [0, cap, min(3, cap - 1), cap]
    nxt = [n_sink, n_sink + (5 % (cap - n_sink)), n_sink, cap - 1]
    c = _paged_case(O, rng, fmt, ofmt, B, Hq, Hkv, [n + steps + 1 for n in n_packed], n_res, cap,
                    layout)
    # the pools hold n_packed[b] + steps + 1 tokens per sequence; the state says n_packed[b]
    st0 = _state([[n_packed[b], n_res[b], nxt[b], 7] for b in range(B)])
    mb = c["tbl"].shape[1]
    print(f"[paged append] bits={bits} hybrid={hybrid} Hq={Hq} Hkv={Hkv} cap={cap} "
          f"sink={n_sink} S={S_} {layout}", flush=True)
    dtbl = _dev(c["tbl"])
    a = [_dev(c["kpool"]), _dev(c["vpool"]), _dev(c["kres"]), _dev(c["vres"]), _dev(st0)]
    bb = [_dev(c["kpool"]), _dev(c["vpool"]), _dev(c["kres"]), _dev(c["vres"])]
    s_in, s_out = _dev(st0), torch.full_like(_dev(st0), -1)
    po_a = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=DEV)
    pl_a = torch.empty((B, Hq, S_), dtype=torch.float32, device=DEV)
    po_b, pl_b = torch.empty_like(po_a), torch.empty_like(pl_a)
    # key-channel factors [B * Hkv][128] (both calls scale q by them the same way)
    norm = (rng.uniform(0.25, 4.0, (B * Hkv, 128)).astype(np.float32) if knorm else None)
    dnorm = _dev(norm) if knorm else None
    for i in range(steps):
        kn = _dev(_f16(rng.standard_normal((B, Hkv, 128)) * 2))
        vn = _dev(_f16(rng.standard_normal((B, Hkv, 128))))
        q = _dev(_f16(rng.standard_normal((B, Hq, 128))))
        K.kvq_append_evict(fmt, kn, vn, a[2], a[3], cap, n_sink, a[0], a[1], c["npool"], c["bs"],
                           c["hs"], dtbl, mb, a[4], B, Hkv)
        K.kvq_decode_attention_paged(fmt, q, B, Hq, Hkv, a[0], a[1], c["npool"], c["bs"], c["hs"],
                                     dtbl, mb, a[4], a[2], a[3], cap, SM, S_, po_a, pl_a,
                                     key_norm=dnorm)
        K.kvq_decode_attention_paged_append(fmt, q, B, Hq, Hkv, bb[0], bb[1], c["npool"], c["bs"],
                                            c["hs"], dtbl, mb, s_in, s_out, bb[2], bb[3], cap,
                                            n_sink, kn, vn, SM, S_, po_b, pl_b, key_norm=dnorm)
        torch.cuda.synchronize()
        assert torch.equal(a[4], s_out), f"state, step {i}"
        assert torch.equal(pl_a, pl_b), f"lse, step {i}"
        assert torch.equal(po_a, po_b), f"partial outputs, step {i}"
        for x, y, what in zip(a[:4], bb, ("K pool", "V pool", "K window", "V window")):
            assert torch.equal(x, y), f"{what}, step {i}"
        s_in, s_out = s_out, s_in
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    K.kvq_combine(po_b, pl_b, B, Hq, 128, S_, out, K.KVQ_OUT_F32)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    if knorm:
        # q' = fp16(q * factor), the binary32 product rounded once to fp16, per channel of
        # the head's kv-head row
        gq = Hq // Hkv
        f = norm.reshape(B, Hkv, 1, 128).repeat(gq, axis=2).reshape(B, Hq, 128)
        qh = (qh.astype(np.float32) * f).astype(np.float16)
    ref = O.attention_paged(ofmt, qh, Hkv, bb[0].cpu().numpy(),
                            bb[1].cpu().numpy(), c["tbl"], s_in.cpu().numpy(), bb[2].cpu().numpy(),
                            bb[3].cpu().numpy(), sm=SM, block_stride=c["bs"], head_stride=c["hs"])
    assert_close(out.cpu().numpy(), ref, "attention after the last step")
