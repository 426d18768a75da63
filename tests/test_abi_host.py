"""Host-only checks of the C ABI: the library loads, exports every call include/kvq.h
declares, and rejects bad arguments before launching anything (these calls never reach a
kernel launch, so they run without a GPU)."""
import ctypes as C
import os
import re

import pytest

from bit_kv_cache_pack_amd import kvq as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

A = 1 << 20          # a fake, 64-byte aligned "device" address (never dereferenced)
MIS = A + 2          # misaligned


def _declared(ret="kvq_status"):
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^" + ret + r"\s+(kvq_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_call():
    names = _declared()
    assert names == sorted(K.EXPORTED)
    sizes = _declared("int64_t")
    assert sizes == sorted(K.EXPORTED_SIZE)
    L = K.lib()
    for n in names + sizes:
        assert hasattr(L, n), n


def _fmt(**kw):
    f = dict(bits=4, head_dim=128, group=32, hybrid=0, block_tokens=128)
    f.update(kw)
    return K.kvq_format(**f)


def _qp(fmt=None, src=A, rows=2, T=256, rs=256 * 128, ts=128, dst=A, dstride=2 * 10240, fb=0):
    f = _fmt() if fmt is None else fmt
    return K.lib().kvq_quantize_pack(C.byref(f) if f is not False else None, src, rows, T, rs, ts,
                                     dst, dstride, fb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=False), K.KVQ_ERR_NULL),
    (dict(fmt=_fmt(bits=5)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(bits=1)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(group=16)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(block_tokens=64)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(hybrid=2)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(head_dim=64)), K.KVQ_ERR_UNSUPPORTED),
    (dict(fmt=_fmt(head_dim=100)), K.KVQ_ERR_SHAPE),
    (dict(src=None), K.KVQ_ERR_NULL),
    (dict(dst=None), K.KVQ_ERR_NULL),
    (dict(rows=0), K.KVQ_ERR_SHAPE),
    (dict(T=100), K.KVQ_ERR_SHAPE),
    (dict(T=0), K.KVQ_ERR_SHAPE),
    (dict(fb=-1), K.KVQ_ERR_SHAPE),
    (dict(ts=64), K.KVQ_ERR_SHAPE),
    (dict(ts=132), K.KVQ_ERR_ALIGN),
    (dict(rs=256 * 128 + 4), K.KVQ_ERR_ALIGN),
    (dict(src=MIS), K.KVQ_ERR_ALIGN),
    (dict(dst=MIS), K.KVQ_ERR_ALIGN),
    (dict(dstride=2 * 10240 + 32), K.KVQ_ERR_ALIGN),
    (dict(dstride=10240), K.KVQ_ERR_SHAPE),          # 2 blocks do not fit
    (dict(fb=1, dstride=2 * 10240), K.KVQ_ERR_SHAPE),
])
def test_quantize_pack_rejects(kw, status):
    assert _qp(**kw) == status


def _dec(fmt=None, q=A, B=1, Hq=8, Hkv=2, kp=A, vp=A, stride=10240, n_packed=128, kr=A, vr=A,
         cap=128, n_res=4, sm=0.088, S=4, po=A, pl=A):
    f = _fmt() if fmt is None else fmt
    return K.lib().kvq_decode_attention(C.byref(f), q, B, Hq, Hkv, kp, vp, stride, n_packed, kr,
                                        vr, cap, n_res, sm, S, po, pl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=_fmt(bits=7)), K.KVQ_ERR_UNSUPPORTED),
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(po=None), K.KVQ_ERR_NULL),
    (dict(pl=None), K.KVQ_ERR_NULL),
    (dict(kp=None), K.KVQ_ERR_NULL),
    (dict(vr=None), K.KVQ_ERR_NULL),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(B=0), K.KVQ_ERR_SHAPE),
    (dict(n_packed=100), K.KVQ_ERR_SHAPE),
    (dict(n_packed=-128), K.KVQ_ERR_SHAPE),
    (dict(n_res=129), K.KVQ_ERR_SHAPE),
    (dict(n_res=-1), K.KVQ_ERR_SHAPE),
    (dict(n_packed=0, n_res=0), K.KVQ_ERR_SHAPE),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(S=1025), K.KVQ_ERR_SHAPE),
    (dict(sm=float("nan")), K.KVQ_ERR_SHAPE),
    (dict(sm=float("inf")), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),   # 17 query heads per kv head
    (dict(stride=10240 + 8), K.KVQ_ERR_ALIGN),
    (dict(n_packed=256), K.KVQ_ERR_SHAPE),          # row stride holds one block only
    (dict(kp=MIS), K.KVQ_ERR_ALIGN),
    (dict(kr=MIS), K.KVQ_ERR_ALIGN),
    (dict(q=MIS), K.KVQ_ERR_ALIGN),
    (dict(po=MIS), K.KVQ_ERR_ALIGN),
])
def test_decode_rejects(kw, status):
    assert _dec(**kw) == status


def _f16(q=A, B=1, Hq=8, Hkv=2, k=A, v=A, stride=1024, n=1000, sm=0.088, S=4, po=A, pl=A):
    return K.lib().kvq_decode_attention_fp16(q, B, Hq, Hkv, k, v, stride, n, sm, S, po, pl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(k=None), K.KVQ_ERR_NULL),
    (dict(pl=None), K.KVQ_ERR_NULL),
    (dict(B=0), K.KVQ_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(n=0), K.KVQ_ERR_SHAPE),
    (dict(stride=999), K.KVQ_ERR_SHAPE),            # stride below n_tokens
    (dict(stride=1025), K.KVQ_ERR_ALIGN),           # odd stride
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(S=1025), K.KVQ_ERR_SHAPE),
    (dict(sm=float("nan")), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(n=1 << 23, stride=1 << 23), K.KVQ_ERR_UNSUPPORTED),   # 2 GiB row
    (dict(k=MIS), K.KVQ_ERR_ALIGN),
    (dict(po=MIS), K.KVQ_ERR_ALIGN),
])
def test_fp16_decode_rejects(kw, status):
    assert _f16(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, A, 1, 8, 128, 4, A, 0), K.KVQ_ERR_NULL),
    ((A, A, 1, 8, 128, 4, None, 0), K.KVQ_ERR_NULL),
    ((A, A, 0, 8, 128, 4, A, 0), K.KVQ_ERR_SHAPE),
    ((A, A, 1, 8, 128, 0, A, 0), K.KVQ_ERR_SHAPE),
    ((A, A, 1, 8, 128, 2000, A, 0), K.KVQ_ERR_SHAPE),
    ((A, A, 1, 8, 64, 4, A, 0), K.KVQ_ERR_UNSUPPORTED),
    ((A, A, 1, 8, 128, 4, A, 3), K.KVQ_ERR_UNSUPPORTED),
    ((MIS, A, 1, 8, 128, 4, A, 0), K.KVQ_ERR_ALIGN),
    ((A, A, 1, 8, 128, 4, MIS, 1), K.KVQ_ERR_ALIGN),
])
def test_combine_rejects(args, status):
    assert K.lib().kvq_combine(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, A, A, A, 1, 2, 128, 128, 0), K.KVQ_ERR_NULL),
    ((A, A, A, A, 1, 2, 128, 128, 128), K.KVQ_ERR_SHAPE),
    ((A, A, A, A, 1, 2, 128, 128, -1), K.KVQ_ERR_SHAPE),
    ((A, A, A, A, 0, 2, 128, 128, 0), K.KVQ_ERR_SHAPE),
    ((A, A, A, A, 1, 2, 96, 128, 0), K.KVQ_ERR_UNSUPPORTED),
    ((A, MIS, A, A, 1, 2, 128, 128, 0), K.KVQ_ERR_ALIGN),
])
def test_append_rejects(args, status):
    assert K.lib().kvq_append_residual(*args, None) == status


def _sr(bufs=(A, A), sizes=(4096, 4096), n=None, sink=A):
    n = len(bufs) if n is None else n
    arr_p = (C.c_void_p * max(1, len(bufs)))(*bufs)
    arr_s = (C.c_int64 * max(1, len(sizes)))(*sizes)
    return K.lib().kvq_stream_read(arr_p, arr_s, n, sink, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bufs=(A, None)), K.KVQ_ERR_NULL),
    (dict(sink=None), K.KVQ_ERR_NULL),
    (dict(n=0), K.KVQ_ERR_SHAPE),
    (dict(bufs=(A,) * 5, sizes=(4096,) * 5), K.KVQ_ERR_SHAPE),
    (dict(sizes=(4096, 0)), K.KVQ_ERR_SHAPE),
    (dict(sizes=(4096, 4100)), K.KVQ_ERR_SHAPE),
    (dict(sizes=(4096, 1 << 62)), K.KVQ_ERR_SHAPE),
    (dict(bufs=(A, A + 8)), K.KVQ_ERR_ALIGN),
    (dict(sink=A + 4), K.KVQ_ERR_ALIGN),
])
def test_stream_read_rejects(kw, status):
    assert _sr(**kw) == status


@pytest.mark.parametrize("bits,hybrid", [(2, 0), (2, 1), (3, 0), (3, 1), (4, 0), (4, 1)])
def test_format_sizes_agree_with_oracle_restatement(oracle_mod, bits, hybrid):
    """The header's size helpers (mirrored in Python) and the oracle's independent
    restatement of the block layout give the same offsets."""
    f = K.Format(bits, 128, bool(hybrid))
    o = oracle_mod.Format(bits, 128, bool(hybrid))
    assert (f.codes_bytes, f.sz_offset, f.sz_bytes, f.flag_offset, f.flag_bytes, f.block_bytes) == \
        (o.codes_bytes, o.sz_offset, o.sz_bytes, o.flag_offset, o.flag_bytes, o.block_bytes)


def test_suggest_splits_bounds():
    for B, Hkv, n in [(1, 8, 32768), (8, 8, 32768), (1, 8, 131072), (64, 40, 4096), (1, 2, 1024),
                      (1, 1, 1)]:
        s = K.suggest_splits(B, Hkv, n)
        assert 1 <= s <= 256
        assert s <= max(1, n // 32 // 8)


def _dec_kn(fmt=None, q=A, norm=A, B=1, Hq=8, Hkv=2, kp=A, vp=A, stride=10240, n_packed=128,
            kr=A, vr=A, cap=128, n_res=4, sm=0.088, S=4, po=A, pl=A):
    f = _fmt() if fmt is None else fmt
    return K.lib().kvq_decode_attention_knorm(C.byref(f), q, norm, B, Hq, Hkv, kp, vp, stride,
                                              n_packed, kr, vr, cap, n_res, sm, S, po, pl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(norm=None), K.KVQ_ERR_NULL),
    (dict(norm=A + 16), K.KVQ_ERR_ALIGN),
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(fmt=_fmt(bits=7)), K.KVQ_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(n_packed=0, n_res=0), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(kp=MIS), K.KVQ_ERR_ALIGN),
])
def test_decode_knorm_rejects(kw, status):
    assert _dec_kn(**kw) == status


def _dec_app(fmt=None, q=A, B=1, Hq=8, Hkv=2, kp=A, vp=A, stride=10240, n_packed=128, kr=A,
             vr=A, cap=128, n_res=4, kn=A, vn=A, sm=0.088, S=4, po=A, pl=A):
    f = _fmt() if fmt is None else fmt
    return K.lib().kvq_decode_attention_append(C.byref(f), q, B, Hq, Hkv, kp, vp, stride,
                                               n_packed, kr, vr, cap, n_res, kn, vn, sm, S, po,
                                               pl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), K.KVQ_ERR_NULL),
    (dict(vn=None), K.KVQ_ERR_NULL),
    (dict(kr=None), K.KVQ_ERR_NULL),
    (dict(vr=None), K.KVQ_ERR_NULL),
    (dict(n_res=0), K.KVQ_ERR_SHAPE),
    (dict(n_res=129), K.KVQ_ERR_SHAPE),
    (dict(kn=A + 16), K.KVQ_ERR_ALIGN),
    (dict(vn=MIS), K.KVQ_ERR_ALIGN),
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(fmt=_fmt(bits=7)), K.KVQ_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(kp=MIS), K.KVQ_ERR_ALIGN),
])
def test_decode_append_rejects(kw, status):
    assert _dec_app(**kw) == status


def _kn(k=A, rows=2, T=300, rs=512 * 128, ts=128, hd=128, norm=A):
    return K.lib().kvq_key_norm(k, rows, T, rs, ts, hd, norm, None)


@pytest.mark.parametrize("kw,status", [
    (dict(norm=None), K.KVQ_ERR_NULL),
    (dict(k=None), K.KVQ_ERR_NULL),
    (dict(rows=0), K.KVQ_ERR_SHAPE),
    (dict(T=-1), K.KVQ_ERR_SHAPE),
    (dict(rs=-8), K.KVQ_ERR_SHAPE),
    (dict(ts=64), K.KVQ_ERR_SHAPE),
    (dict(hd=64, ts=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(ts=132), K.KVQ_ERR_ALIGN),
    (dict(rs=512 * 128 + 4), K.KVQ_ERR_ALIGN),
    (dict(k=MIS), K.KVQ_ERR_ALIGN),
    (dict(norm=A + 32), K.KVQ_ERR_ALIGN),
    (dict(rows=1 << 40), K.KVQ_ERR_SHAPE),
])
def test_key_norm_rejects(kw, status):
    assert _kn(**kw) == status


def _cs(x=A, rows=2, T=300, xrs=512 * 128, xts=128, hd=128, norm=A, rpn=1, mode=0, y=A,
        yrs=512 * 128, yts=128):
    return K.lib().kvq_channel_scale(x, rows, T, xrs, xts, hd, norm, rpn, mode, y, yrs, yts, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), K.KVQ_ERR_NULL),
    (dict(norm=None), K.KVQ_ERR_NULL),
    (dict(y=None), K.KVQ_ERR_NULL),
    (dict(rows=0), K.KVQ_ERR_SHAPE),
    (dict(T=-5), K.KVQ_ERR_SHAPE),
    (dict(rpn=0), K.KVQ_ERR_SHAPE),
    (dict(xts=120), K.KVQ_ERR_SHAPE),
    (dict(yts=0), K.KVQ_ERR_SHAPE),
    (dict(yrs=-8), K.KVQ_ERR_SHAPE),
    (dict(hd=256, xts=256, yts=256), K.KVQ_ERR_UNSUPPORTED),
    (dict(mode=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(xts=136 + 2), K.KVQ_ERR_ALIGN),
    (dict(yrs=512 * 128 + 2), K.KVQ_ERR_ALIGN),
    (dict(x=MIS), K.KVQ_ERR_ALIGN),
    (dict(y=MIS), K.KVQ_ERR_ALIGN),
    (dict(norm=A + 4), K.KVQ_ERR_ALIGN),
    (dict(rows=1 << 40, T=1 << 20), K.KVQ_ERR_SHAPE),
])
def test_channel_scale_rejects(kw, status):
    assert _cs(**kw) == status


BB4 = 10240          # 4-bit block bytes


def _pool_kw(**kw):
    d = dict(pool_blocks=10, bs=2 * BB4, hs=BB4, tbl=A, maxb=4)
    d.update(kw)
    return d


def _ptp(fmt=None, src=A, B=2, Hkv=2, rs=256 * 128, ts=128, cnt=A, st=A, maxc=256, pool=A, **kw):
    f = _fmt() if fmt is None else fmt
    p = _pool_kw(**kw)
    return K.lib().kvq_pack_tokens_paged(C.byref(f), src, B, Hkv, rs, ts, cnt, st, maxc, pool,
                                         p["pool_blocks"], p["bs"], p["hs"], p["tbl"], p["maxb"],
                                         None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=_fmt(bits=1)), K.KVQ_ERR_UNSUPPORTED),
    (dict(src=None), K.KVQ_ERR_NULL),
    (dict(cnt=None), K.KVQ_ERR_NULL),
    (dict(st=None), K.KVQ_ERR_NULL),
    (dict(pool=None), K.KVQ_ERR_NULL),
    (dict(tbl=None), K.KVQ_ERR_NULL),
    (dict(B=0), K.KVQ_ERR_SHAPE),
    (dict(maxc=-1), K.KVQ_ERR_SHAPE),
    (dict(ts=64), K.KVQ_ERR_SHAPE),
    (dict(ts=132), K.KVQ_ERR_ALIGN),
    (dict(src=MIS), K.KVQ_ERR_ALIGN),
    (dict(pool=MIS), K.KVQ_ERR_ALIGN),
    (dict(pool_blocks=0), K.KVQ_ERR_SHAPE),
    (dict(maxb=0), K.KVQ_ERR_SHAPE),
    (dict(bs=2 * BB4 + 32), K.KVQ_ERR_ALIGN),
    (dict(hs=BB4 - 64), K.KVQ_ERR_SHAPE),             # heads of a block overlap
    (dict(bs=BB4, hs=BB4), K.KVQ_ERR_SHAPE),          # blocks overlap the next head
    (dict(maxb=1 << 24), K.KVQ_ERR_SHAPE),
])
def test_pack_tokens_paged_rejects(kw, status):
    assert _ptp(**kw) == status


def test_pack_tokens_paged_accepts_both_pool_layouts():
    # [blocks][Hkv][bb] and [Hkv][blocks][bb]; max_count 0 launches nothing
    assert _ptp(maxc=0) == K.KVQ_OK
    assert _ptp(maxc=0, bs=BB4, hs=10 * BB4) == K.KVQ_OK


def _ae(fmt=None, kn=A, vn=A, kr=A, vr=A, cap=128, sink=4, kp=A, vp=A, state=A, B=2, Hkv=2, **kw):
    f = _fmt() if fmt is None else fmt
    p = _pool_kw(**kw)
    return K.lib().kvq_append_evict(C.byref(f), kn, vn, kr, vr, cap, sink, kp, vp,
                                    p["pool_blocks"], p["bs"], p["hs"], p["tbl"], p["maxb"],
                                    state, B, Hkv, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), K.KVQ_ERR_NULL),
    (dict(vp=None), K.KVQ_ERR_NULL),
    (dict(state=None), K.KVQ_ERR_NULL),
    (dict(tbl=None), K.KVQ_ERR_NULL),
    (dict(cap=0), K.KVQ_ERR_SHAPE),
    (dict(sink=128), K.KVQ_ERR_SHAPE),
    (dict(sink=-1), K.KVQ_ERR_SHAPE),
    (dict(B=0), K.KVQ_ERR_SHAPE),
    (dict(state=A + 16), K.KVQ_ERR_ALIGN),
    (dict(kr=MIS), K.KVQ_ERR_ALIGN),
    (dict(hs=64), K.KVQ_ERR_SHAPE),
    (dict(fmt=_fmt(group=16)), K.KVQ_ERR_UNSUPPORTED),
])
def test_append_evict_rejects(kw, status):
    assert _ae(**kw) == status


def _dp(fmt=None, q=A, B=2, Hq=8, Hkv=2, kp=A, vp=A, state=A, kr=A, vr=A, cap=128, kn=None,
        sm=0.088, S=4, po=A, pl=A, **kw):
    f = _fmt() if fmt is None else fmt
    p = _pool_kw(**kw)
    return K.lib().kvq_decode_attention_paged(C.byref(f), q, B, Hq, Hkv, kp, vp,
                                              p["pool_blocks"], p["bs"], p["hs"], p["tbl"],
                                              p["maxb"], state, kr, vr, cap, kn, sm, S, po, pl,
                                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(state=None), K.KVQ_ERR_NULL),
    (dict(kr=None), K.KVQ_ERR_NULL),
    (dict(tbl=None), K.KVQ_ERR_NULL),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(cap=0), K.KVQ_ERR_SHAPE),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(sm=float("nan")), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(po=MIS), K.KVQ_ERR_ALIGN),
    (dict(state=A + 16), K.KVQ_ERR_ALIGN),
    (dict(bs=3 * BB4 + 16), K.KVQ_ERR_ALIGN),
    (dict(pool_blocks=0), K.KVQ_ERR_SHAPE),
    (dict(fmt=_fmt(bits=6)), K.KVQ_ERR_UNSUPPORTED),
    (dict(kn=A + 8), K.KVQ_ERR_ALIGN),
])
def test_decode_paged_rejects(kw, status):
    assert _dp(**kw) == status


def _dpa(fmt=None, q=A, B=2, Hq=8, Hkv=2, kp=A, vp=A, state=A, state_out=A + 4096, kr=A, vr=A,
         cap=128, sink=4, knew=A, vnew=A, kn=None, sm=0.088, S=4, po=A, pl=A, **kw):
    f = _fmt() if fmt is None else fmt
    p = _pool_kw(**kw)
    return K.lib().kvq_decode_attention_paged_append(
        C.byref(f), q, B, Hq, Hkv, kp, vp, p["pool_blocks"], p["bs"], p["hs"], p["tbl"],
        p["maxb"], state, state_out, kr, vr, cap, sink, knew, vnew, kn, sm, S, po, pl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(knew=None), K.KVQ_ERR_NULL),
    (dict(vnew=None), K.KVQ_ERR_NULL),
    (dict(state_out=None), K.KVQ_ERR_NULL),
    (dict(state=None), K.KVQ_ERR_NULL),
    (dict(sink=-1), K.KVQ_ERR_SHAPE),
    (dict(sink=128), K.KVQ_ERR_SHAPE),
    (dict(state_out=A), K.KVQ_ERR_SHAPE),                 # the same buffer
    (dict(state_out=A + 64, B=5), K.KVQ_ERR_SHAPE),      # overlapping (5 states = 80 bytes)
    (dict(state_out=A + 4096 + 16), K.KVQ_ERR_ALIGN),
    (dict(knew=A + 8), K.KVQ_ERR_ALIGN),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(tbl=None), K.KVQ_ERR_NULL),
])
def test_decode_paged_append_rejects(kw, status):
    assert _dpa(**kw) == status


def test_suggest_splits_paged_bounds():
    assert K.suggest_splits_paged(0, 0, 8) == 1
    # 16 sequences of 1.5K..32K tokens, 8 kv heads: 16 splits
    assert K.suggest_splits_paged(270520, 31712, 8) == 16
    for total, mx, hkv in [(32640, 32640, 8), (10 ** 7, 4096, 40), (100, 100, 1), (5000, 300, 2)]:
        s = K.suggest_splits_paged(total, mx, hkv)
        assert 1 <= s <= 256 and s <= max(1, mx // 256)


def test_outer_calls_reject_hybrid_and_bad_shapes():
    L = K.lib()
    hyb = _fmt(hybrid=1)
    assert L.kvq_quantize_pack_outer(C.byref(hyb), A, 2, 256, 256 * 128, 128, A, 2 * 10240, 0,
                                     None) == K.KVQ_ERR_UNSUPPORTED
    f = _fmt()
    assert L.kvq_quantize_pack_outer(C.byref(f), None, 2, 256, 256 * 128, 128, A, 2 * 10240, 0,
                                     None) == K.KVQ_ERR_NULL
    assert L.kvq_quantize_pack_outer(C.byref(f), A, 2, 100, 256 * 128, 128, A, 2 * 10240, 0,
                                     None) == K.KVQ_ERR_SHAPE
    assert L.kvq_decode_attention_outer(C.byref(hyb), A, 1, 8, 2, A, A, 10240, 128, A, A, 128, 4,
                                        0.088, 4, A, A, None) == K.KVQ_ERR_UNSUPPORTED
    assert L.kvq_decode_attention_outer(C.byref(f), A, 1, 6, 4, A, A, 10240, 128, A, A, 128, 4,
                                        0.088, 4, A, A, None) == K.KVQ_ERR_SHAPE
    assert L.kvq_decode_attention_outer(C.byref(f), MIS, 1, 8, 2, A, A, 10240, 128, A, A, 128, 4,
                                        0.088, 4, A, A, None) == K.KVQ_ERR_ALIGN


def test_split_rules_match_the_header(tmp_path):
    """The Python mirrors of the header's inline split rules give the same counts as the
    header itself, compiled with the host C compiler, over a grid of shapes."""
    import itertools
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    shapes = list(itertools.product([1, 2, 8, 16, 64], [1, 2, 8, 40], [1, 1024, 4096, 32768, 131072],
                                    [128, 256]))
    paged = list(itertools.product([1, 5000, 270520, 4 << 20], [1, 1000, 31712, 131072], [1, 8],
                                   [128, 256]))
    src = tmp_path / "rules.c"
    lines = ['#include <stdio.h>', '#include "kvq.h"', "int main(void) {"]
    lines += [f'printf("%d\\n", kvq_suggest_splits({B}, {H}, {n}, {cu}));' for B, H, n, cu in shapes]
    lines += [f'printf("%d\\n", kvq_suggest_splits_paged({t}LL, {m}, {H}, {cu}));'
              for t, m, H, cu in paged]
    lines += ["return 0; }"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "rules"
    subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                    "-I", "/opt/rocm/include", "-o", str(exe), str(src)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [K.suggest_splits(B, H, n, cu) for B, H, n, cu in shapes]
    want += [K.suggest_splits_paged(t, m, H, cu) for t, m, H, cu in paged]
    assert got == want


def test_split_rule_on_the_workloads():
    """One wide workgroup per CU for few rows, else three 4-wave workgroups per CU (plus
    the window's split) where splits stay long and two where they would get short; the
    8-tile floor for short sequences."""
    import synth_inputs as S
    got = {n: K.suggest_splits(w.B, w.Hkv, w.L) for n, w in S.WORKLOADS.items()}
    assert got == {"tiny": 4, "llama8b_32k": 32, "batch8_2bit_hybrid": 13,
                   "long_128k_3bit": 32, "mha_b64_append": 1}
    # three per CU: 64 rows -> 12 packed splits + the window's; 8 rows of 256K tokens ->
    # 96 + 1; one split (2560 rows) stays one
    assert K.suggest_splits(8, 8, 32768) == 13
    assert K.suggest_splits(1, 8, 262144) == 97
    assert K.suggest_splits(64, 40, 4096) == 1
    # the wide branch: 32 rows on 256 CUs, 8 splits of 128 tiles; one tile more per split
    # leaves it for the per-CU rules (two per CU: 16 splits)
    assert K.suggest_splits(4, 8, 32768) == 8
    assert K.suggest_splits(4, 8, 32768 + 8 * 32) == 16


# ---- the fused decode (split merge inside the launch) ------------------------------------

def _ws_bytes(B, Hq, Hkv, S):
    """The header's workspace size: per (batch, kv-head, chunk of <= 4 query heads) one
    2080-byte slot per node below the root of the fan-in-32 split tree."""
    slots = 0
    n = S
    while n > 1:
        slots += n
        n = (n + 31) // 32
    return B * Hkv * ((Hq // Hkv + 3) // 4) * slots * 2080


@pytest.mark.parametrize("B,Hq,Hkv,S", [(1, 32, 8, 1), (1, 32, 8, 64), (8, 32, 8, 12),
                                         (1, 8, 2, 9), (2, 40, 40, 3), (1, 10, 2, 1024),
                                         (3, 48, 3, 513)])
def test_decode_workspace_bytes(B, Hq, Hkv, S):
    assert K.kvq_decode_workspace_bytes(B, Hq, Hkv, S) == _ws_bytes(B, Hq, Hkv, S)


def test_decode_workspace_bytes_known_values():
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 1) == 0
    # 8 rows x 1 chunk; S = 64: 64 + 2 slots; S = 32: 32 slots (one level)
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 64) == 8 * 66 * 2080
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 32) == 8 * 32 * 2080
    for bad in [(0, 8, 2, 4), (1, 8, 3, 4), (1, 8, 2, 0), (1, 8, 2, 1025)]:
        assert K.lib().kvq_decode_workspace_bytes(*bad) == -1


W = 1 << 24          # a fake, 256-byte aligned workspace address


def _fused(fmt=None, q=A, kn=None, B=1, Hq=8, Hkv=2, kp=A, vp=A, stride=10240, n_packed=128,
           kr=A, vr=A, cap=128, n_res=4, knew=None, vnew=None, sm=0.088, S=4, ws=W,
           wsb=1 << 20, out=A, od=K.KVQ_OUT_F32):
    f = _fmt() if fmt is None else fmt
    return K.lib().kvq_decode_attention_fused(C.byref(f), q, kn, B, Hq, Hkv, kp, vp, stride,
                                              n_packed, kr, vr, cap, n_res, knew, vnew, sm, S, ws,
                                              wsb, out, od, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=_fmt(bits=7)), K.KVQ_ERR_UNSUPPORTED),
    (dict(q=None), K.KVQ_ERR_NULL),
    (dict(out=None), K.KVQ_ERR_NULL),
    (dict(ws=None), K.KVQ_ERR_NULL),
    (dict(kp=None), K.KVQ_ERR_NULL),
    (dict(knew=A), K.KVQ_ERR_NULL),                 # k_new without v_new
    (dict(knew=A, vnew=A, kr=None), K.KVQ_ERR_NULL),
    (dict(knew=A, vnew=A, n_res=0), K.KVQ_ERR_SHAPE),
    (dict(knew=MIS, vnew=A), K.KVQ_ERR_ALIGN),
    (dict(kn=MIS), K.KVQ_ERR_ALIGN),
    (dict(od=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(out=MIS), K.KVQ_ERR_ALIGN),
    (dict(ws=W + 64), K.KVQ_ERR_ALIGN),             # 64-byte but not 256-byte aligned
    (dict(wsb=_ws_bytes(1, 8, 2, 4) - 1), K.KVQ_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), K.KVQ_ERR_SHAPE),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    (dict(S=1025), K.KVQ_ERR_SHAPE),
    (dict(n_packed=0, n_res=0), K.KVQ_ERR_SHAPE),
    (dict(sm=float("nan")), K.KVQ_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), K.KVQ_ERR_UNSUPPORTED),
    (dict(q=MIS), K.KVQ_ERR_ALIGN),
])
def test_decode_fused_rejects(kw, status):
    assert _fused(**kw) == status


def test_decode_fused_one_split_needs_no_workspace():
    """With one split nothing is merged: a NULL workspace of size 0 passes validation (the
    call then launches, so only the rejection of a bad out pointer is checked here)."""
    assert _fused(S=1, ws=None, wsb=0, out=MIS) == K.KVQ_ERR_ALIGN
    assert _fused(S=2, ws=None, wsb=0, out=A) == K.KVQ_ERR_NULL


def _noalloc(B=1, Hq=8, Hkv=2, n_packed=128, S=4, out=A, od=K.KVQ_OUT_F32, knew=None, vnew=None):
    f = _fmt()
    return K.lib().kvq_decode_attention_fused_noalloc(C.byref(f), A, None, B, Hq, Hkv, A, A,
                                                      10240 * 256, n_packed, A, A, 128, 4, knew,
                                                      vnew, 0.088, S, out, od, None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), K.KVQ_ERR_NULL),
    (dict(out=MIS), K.KVQ_ERR_ALIGN),
    (dict(od=5), K.KVQ_ERR_UNSUPPORTED),
    (dict(knew=A), K.KVQ_ERR_NULL),
    (dict(S=0), K.KVQ_ERR_SHAPE),
    # 8 rows of 4 query heads at 1024 splits need 17.6 MB of records: more than the scratch
    (dict(B=1, Hq=32, Hkv=8, n_packed=32768, S=1024), K.KVQ_ERR_TOO_LARGE),
])
def test_decode_fused_noalloc_rejects(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == K.KVQ_NOALLOC_SCRATCH_BYTES
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 1024) > K.KVQ_NOALLOC_SCRATCH_BYTES
    assert K.kvq_decode_workspace_bytes(1, 32, 8, 64) <= K.KVQ_NOALLOC_SCRATCH_BYTES
