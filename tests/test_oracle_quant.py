"""Pins of the oracle's quantizer, packer and block layout against things other than itself.

- fp16 conversion: numpy's float16 cast (a library routine) on every bit pattern and on
  random, tie and overflow values;
- hand-worked examples (tests/golden/quant_hand_examples.json, derived from the pages'
  formulas by hand);
- brute force: every code is the level nearest to x among all 2^b levels;
- invariants: code range, min -> code 0, max -> code N, error <= scale/2, exact minimum;
- packing: an independent Python big-int packer;
- block layout: rebuilt in Python from the group results and the stated offsets.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth_inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_hand_examples.json")


# ------------------------------------------------------------------------------ fp16 --

def test_f16_to_f32_all_bit_patterns(oracle_mod):
    O = oracle_mod
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_matches_numpy(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(3000).astype(np.float32) * np.float32(s) for s in
            (1e-8, 1e-6, 1e-4, 1e-2, 1, 100, 3e4, 7e4)]
    # exact ties between neighbouring fp16 values (normal and subnormal) and overflow edges
    h = np.arange(0, 0x7bff, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    edges = np.array([65504, 65519.99, 65520, 65536, 2 ** -25, 2 ** -24, 3 * 2 ** -26,
                      2 ** -14, 2 ** -14 - 2 ** -25, 0.0, -0.0, 1 / 15, 2 / 3], np.float32)
    allv = np.concatenate(vals + [ties, -ties, edges, -edges])
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(x)) for x in allv], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ hand examples ----

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def _golden_input(ex):
    if "x_bits" in ex:
        bits = [int(b, 16) for b in ex["x_bits"]]
        bits += [int(ex["fill_bits"], 16)] * (32 - len(bits))
        return np.array(bits, np.uint16).view(np.float16)
    x = list(ex["x"]) + [ex["fill"]] * (32 - len(ex["x"]))
    return np.array(x, np.float32).astype(np.float16)


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_examples(oracle_mod, ex):
    O = oracle_mod
    x = _golden_input(ex)
    r = O.quantize_group(x, ex["bits"], ex["hybrid"])
    codes = list(ex["codes"]) + [ex["codes_fill"]] * (32 - len(ex["codes"]))
    assert r.scale == int(ex["scale"], 16), hex(r.scale)
    assert r.zero == int(ex["zero"], 16), hex(r.zero)
    assert list(r.codes) == codes
    assert r.flag == ex["flag"]


# ---------------------------------------------------------------- brute force -------

def _levels(scale_bits, zero_bits, bits):
    s = float(np.uint16(scale_bits).view(np.float16))
    z = float(np.uint16(zero_bits).view(np.float16))
    return z + np.arange(2 ** bits, dtype=np.float64) * s, s, z


KINDS = ["normal", "t5", "wide", "tiny", "offset", "few_levels", "ternary"]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_asym_codes_are_nearest_level(oracle_mod, bits, kind):
    O = oracle_mod
    rng = np.random.default_rng(100 + bits)
    groups = S.random_groups(rng, 300, kind)
    N = 2 ** bits - 1
    for x16 in groups:
        r = O.quantize_group(x16, bits)
        lv, s, z = _levels(r.scale, r.zero, bits)
        x = x16.astype(np.float64)
        if s == 0.0:
            assert np.all(r.codes == 0)
            continue
        dist = np.abs(x[:, None] - lv[None, :])
        best = dist.min(axis=1)
        got = dist[np.arange(32), r.codes]
        # nearest level; fp32 evaluation of t may only matter at an exact-tie margin
        assert np.all(got <= best + 1e-6 * s)
        # exact ties (equal distance to two levels) resolve to the upper code
        for i in range(32):
            ties = np.flatnonzero(np.abs(dist[i] - best[i]) <= 0.0)
            if len(ties) == 2:
                assert r.codes[i] == ties.max()
        assert r.codes.max() <= N


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_asym_invariants(oracle_mod, bits, kind):
    O = oracle_mod
    rng = np.random.default_rng(200 + bits)
    N = 2 ** bits - 1
    for x16 in S.random_groups(rng, 300, kind):
        r = O.quantize_group(x16, bits)
        lv, s, z = _levels(r.scale, r.zero, bits)
        x = x16.astype(np.float64)
        xhat = lv[r.codes]
        assert z == x.min()                      # zero = min, exact
        if s == 0.0:
            assert np.all(np.abs(x - xhat) <= 2.0 ** -20)
            continue
        assert r.codes[np.argmin(x)] == 0
        if s >= 2.0 ** -14:     # fp16-normal scale: relative rounding <= 2^-11
            assert r.codes[np.argmax(x)] == N
        # round-trip error <= scale/2 (the pages' bound); when the fp16 scale is rounded
        # down, the clipped top of the range adds N * (range/N - scale), which only
        # exceeds scale/2 when the scale is an fp16 subnormal (absolute rounding 2^-25)
        clip = max(0.0, (x.max() - x.min()) - N * s)
        assert np.all(np.abs(x - xhat) <= max(0.5 * s, clip) + s * 2.0 ** -16)
        if s >= 2.0 ** -14:
            assert clip <= 0.5 * s
            assert np.all(np.abs(x - xhat) <= s * (0.5 + 2.0 ** -16))
        assert xhat[np.argmin(x)] == x.min()
        # the stored scale is the fp16 rounding of the fp32 quotient (numpy float ops)
        sf = (np.float32(x.max()) - np.float32(x.min())) / np.float32(N)
        assert r.scale == int(np.float16(sf).view(np.uint16))


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=0x7bff), min_size=32, max_size=32),
       st.lists(st.booleans(), min_size=32, max_size=32), st.sampled_from([2, 3, 4]))
def test_asym_property_random_bit_patterns(oracle_mod, mags, signs, bits):
    O = oracle_mod
    h = np.array([m | (0x8000 if s else 0) for m, s in zip(mags, signs)], np.uint16)
    x16 = h.view(np.float16)
    r = O.quantize_group(x16, bits)
    lv, s, z = _levels(r.scale, r.zero, bits)
    x = x16.astype(np.float64)
    assert 0 <= r.codes.min() and r.codes.max() <= 2 ** bits - 1
    if s > 0:
        N = 2 ** bits - 1
        clip = max(0.0, (x.max() - x.min()) - N * s)
        assert np.all(np.abs(x - lv[r.codes]) <= max(0.5 * s, clip) + s * 2.0 ** -16)
    # deterministic
    r2 = O.quantize_group(x16, bits)
    assert r2.scale == r.scale and r2.zero == r.zero and np.array_equal(r2.codes, r.codes)


# ------------------------------------------------------------------ hybrid ----------

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_sym_candidate_nearest_on_signed_grid(oracle_mod, bits, kind):
    O = oracle_mod
    rng = np.random.default_rng(300 + bits)
    off = 2 ** (bits - 1)
    Qs = off - 1
    for x16 in S.random_groups(rng, 200, kind):
        r, ok = O.sym_candidate(x16, bits)
        x = x16.astype(np.float64)
        s = float(np.uint16(r.scale).view(np.float16))
        assert r.scale == int(np.float16(np.float32(np.abs(x).max()) / np.float32(Qs)).view(np.uint16))
        if not ok:
            continue
        z = float(np.uint16(r.zero).view(np.float16))
        assert z == -off * s
        k = r.codes.astype(np.int64) - off
        assert np.all(np.abs(k) <= Qs)
        if s == 0:
            assert np.all(k == 0)
            continue
        grid = np.arange(-Qs, Qs + 1, dtype=np.float64) * s
        dist = np.abs(x[:, None] - grid[None, :])
        got = np.abs(x - k * s)
        assert np.all(got <= dist.min(axis=1) + 1e-6 * s)
        # decodes with the same formula as asym: zero + code * scale
        assert np.allclose(z + r.codes * s, k * s, rtol=0, atol=0)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_hybrid_flag_follows_lower_error(oracle_mod, bits, kind):
    O = oracle_mod
    rng = np.random.default_rng(400 + bits)
    n_sym = 0
    groups = S.random_groups(rng, 300, kind)
    for x16 in groups:
        r = O.quantize_group(x16, bits, hybrid=True)
        a = O.asym_candidate(x16, bits)
        sy, ok = O.sym_candidate(x16, bits)
        x = x16.astype(np.float64)

        def sse64(c):
            s = float(np.uint16(c.scale).view(np.float16))
            z = float(np.uint16(c.zero).view(np.float16))
            return float(np.sum((x - (z + c.codes * s)) ** 2))

        ea, es = sse64(a), (sse64(sy) if ok else np.inf)
        chosen = sy if r.flag == 0 else a
        assert (r.scale, r.zero) == (chosen.scale, chosen.zero)
        assert np.array_equal(r.codes, chosen.codes)
        gap = abs(ea - es) / max(ea, es, 1e-300)
        if np.isfinite(es) and gap > 1e-5:
            assert r.flag == (0 if es < ea else 1)
        if not ok:
            assert r.flag == 1
        n_sym += r.flag == 0
    # groups on a symmetric ternary grid {-a, 0, a} are exact in the symmetric mode
    if kind == "ternary":
        assert n_sym > 0.9 * len(groups)


def test_group_sse_pairwise_order(oracle_mod):
    """The fp32 error sum is a balanced tree in channel order: a case where a sequential
    fp32 sum gives a different float pins the order."""
    O = oracle_mod
    x = np.zeros(32, np.float16)
    x[0] = 2048.0
    x[1:] = 0.5
    codes = np.zeros(32, np.uint8)
    got = O.group_sse(x, codes, 0x0000, 0x0000)   # scale 0, zero 0: e = x
    e2 = (x.astype(np.float32)) ** 2
    v = list(e2)
    w = 1
    while w < 32:
        v = [np.float32(v[i] + v[i + 1]) for i in range(0, len(v), 2)]
        w *= 2
    seq = np.float32(0)
    for t in e2:
        seq = np.float32(seq + t)
    assert got == v[0]
    assert v[0] != seq


# ------------------------------------------------------------------ packing ---------

def _bigint_pack(codes, bits):
    w = 0
    for i, c in enumerate(codes):
        w |= int(c) << (bits * i)
    return w.to_bytes(32 * bits // 8, "little")


def _bigint_unpack(data, bits):
    w = int.from_bytes(data, "little")
    return [(w >> (bits * i)) & ((1 << bits) - 1) for i in range(32)]


@settings(max_examples=300, deadline=None)
@given(st.sampled_from([2, 3, 4]), st.data())
def test_pack_matches_bigint(oracle_mod, bits, data):
    O = oracle_mod
    codes = data.draw(st.lists(st.integers(0, 2 ** bits - 1), min_size=32, max_size=32))
    packed = O.pack_codes(np.array(codes, np.uint8), bits)
    assert packed == _bigint_pack(codes, bits)
    assert list(O.unpack_codes(packed, bits)) == codes
    assert _bigint_unpack(packed, bits) == codes


def test_three_bit_codes_straddle_words(oracle_mod):
    O = oracle_mod
    codes = np.zeros(32, np.uint8)
    codes[10] = 7        # bits 30..32: crosses the first 32-bit word
    codes[21] = 7        # bits 63..65: crosses the second
    p = np.frombuffer(O.pack_codes(codes, 3), np.uint32)
    assert p[0] == 0xC0000000 and p[1] == 0x80000001 and p[2] == 0x00000003


# ------------------------------------------------------------------ block layout ----

@pytest.mark.parametrize("bits,hybrid", [(4, False), (3, False), (2, False), (2, True),
                                         (4, True), (3, True)])
def test_block_layout_rebuilt_in_python(oracle_mod, bits, hybrid):
    O = oracle_mod
    fmt = O.Format(bits, 128, hybrid)
    codes_bytes = 128 * 128 * bits // 8
    assert fmt.codes_bytes == codes_bytes
    assert fmt.sz_offset == codes_bytes            # already 64-B aligned at head_dim 128
    assert fmt.sz_bytes == 128 * 4 * 4
    assert fmt.flag_offset == codes_bytes + 2048
    assert fmt.block_bytes == codes_bytes + 2048 + (64 if hybrid else 0)
    rng = np.random.default_rng(7)
    rows, T = 3, 256
    src = S.random_groups(rng, rows * T * 4, "t5").reshape(rows, T, 128)
    packed = O.quantize_pack(fmt, src)
    bb = fmt.block_bytes
    assert packed.shape == (rows, 2 * bb)
    gb = 4 * bits
    for r in range(rows):
        for t in range(0, T, 17):
            blk = packed[r, (t // 128) * bb:(t // 128 + 1) * bb].tobytes()
            tb = t % 128
            for g in range(4):
                gr = O.quantize_group(src[r, t, 32 * g:32 * g + 32], bits, hybrid)
                off = tb * 4 * gb + g * gb
                assert blk[off:off + gb] == _bigint_pack(gr.codes, bits)
                so = fmt.sz_offset + (tb * 4 + g) * 4
                assert int.from_bytes(blk[so:so + 2], "little") == gr.scale
                assert int.from_bytes(blk[so + 2:so + 4], "little") == gr.zero
                if hybrid:
                    bit = tb * 4 + g
                    byte = blk[fmt.flag_offset + bit // 8]
                    assert (byte >> (bit % 8)) & 1 == gr.flag


def test_quantize_pack_first_block_and_strides(oracle_mod):
    """Writing blocks at an offset leaves the others untouched (the append/flush case)."""
    O = oracle_mod
    fmt = O.Format(4)
    rng = np.random.default_rng(8)
    src = S.random_groups(rng, 2 * 384 * 4, "normal").reshape(2, 384, 128)
    full = O.quantize_pack(fmt, src)
    part = np.zeros_like(full)
    O.quantize_pack(fmt, src[:, :256], dst=part)
    O.quantize_pack(fmt, np.ascontiguousarray(src[:, 256:]), first_block=2, dst=part)
    assert np.array_equal(part, full)


def test_dequant_reads_layout(oracle_mod):
    O = oracle_mod
    for bits, hybrid in [(4, False), (3, False), (2, True)]:
        fmt = O.Format(bits, 128, hybrid)
        rng = np.random.default_rng(9)
        src = S.random_groups(rng, 2 * 128 * 4, "normal").reshape(2, 128, 128)
        packed = O.quantize_pack(fmt, src)
        deq = O.dequant(fmt, packed, 128)
        for r in range(2):
            for t in (0, 5, 127):
                for g in range(4):
                    gr = O.quantize_group(src[r, t, 32 * g:32 * g + 32], bits, hybrid)
                    lv, s, z = _levels(gr.scale, gr.zero, bits)
                    assert np.array_equal(deq[r, t, 32 * g:32 * g + 32], lv[gr.codes])
