"""Benchmark of the packed low-bit KV decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step = kvq_decode_attention + kvq_combine over the whole cache of the workload (the
decode-attention step the metric names). Inputs are resident in HBM before timing starts.
The steps are launched back to back from Python; the same steps replayed from a captured
HIP graph are reported next to them, and the same K steps timed once more after the other
headline measurements ("us_per_step_repeat": a check that the clock had settled).
To keep the 256 MB Infinity Cache (MALL) from serving the reads, the timed loop rotates
over enough independent copies of the packed cache to exceed 512 MB. Also measured, and
reported next to the step: the flush (kvq_quantize_pack of the 128-token window of every
row), the one-token append, the key-channel normalization passes over the prefill keys and
the decode step with normalized queries, the FP16 flash-decoding baseline, the same step
over outer-dimension (KIVI-style) groups, a serving-shaped paged batch, a plain device copy
and a plain streaming read of the step's bytes (same rotation) as bandwidth references, the
CPU oracle on a bounded sample of the same workload (all host threads, and one thread), and,
under "per_config", the step and decode figures of the other workloads (with the share of
symmetric-mode groups for the hybrid cache, and the flush and amortized serving step where
the window is full).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + effective KV GB/s (% HBM peak), L=32K 4-bit GQA"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's suggestion")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-fp16-baseline", action="store_true")
    ap.add_argument("--no-key-norm", action="store_true")
    ap.add_argument("--no-paged", action="store_true")
    ap.add_argument("--no-outer", action="store_true")
    ap.add_argument("--paged-workload", default="paged_ragged_b16")
    ap.add_argument("--paged-splits", type=int, default=0, help="0 = the library's suggestion")
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated by the timed loop (0 = enough to exceed 512 MB)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other workloads' step / decode figures")
    ap.add_argument("--per-config-steps", type=int, default=200)
    ap.add_argument("--cpu-single-seconds", type=float, default=3.0)
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("decode_attn.hip", "decode_common.h", "kvq_device.h"):
        with open(os.path.join(ROOT, "bit_kv_cache_pack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was
    taken on the current decode kernel source."""
    p = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m = re.search(r"kernel_source_digest:\s*(\w+)", txt)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_source_digest():
        return None
    return float(t.group(1))


def cpu_baseline(wl, x, seconds: float, single_seconds: float):
    """The CPU oracle (fp64 dequant + attention), as it stands, on the host cores."""
    import numpy as np
    from oracle import oracle as O
    rows = wl.B * wl.Hkv
    fmt = O.Format(wl.bits, 128, wl.hybrid)
    kps, vps = x.packed_src()
    kp = O.quantize_pack(fmt, np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128)))
    vp = O.quantize_pack(fmt, np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128)))
    kr, vr = x.residual()
    threads = O.default_threads()

    def run(n_threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            O.attention(fmt, x.q, wl.Hkv, kp, vp, wl.n_packed, kr, vr, wl.n_res,
                        n_threads=n_threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    reps, el = run(threads, seconds)
    step_s = el / reps
    reps1, el1 = run(1, single_seconds)
    return {"value": round(wl.step_bytes() / step_s / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "ms_per_step": round(step_s * 1e3, 3),
            "single_thread_ms_per_step": round(el1 / reps1 * 1e3, 3),
            "single_thread_GB_per_s": round(wl.step_bytes() / (el1 / reps1) / 1e9, 4),
            "cpu_model": cpu_model(),
            "sample": f"{reps} full decode steps of {wl.name} (all {wl.B * wl.Hq} heads, "
                      f"{wl.L} tokens; dequantize + fp64 softmax attention) on {threads} "
                      f"threads, {el:.1f} s; {reps1} steps on one thread, {el1:.1f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def flag_sym_ratio(fmt, caches_kv, rows, nb):
    """Share of groups the hybrid quantizer stored in symmetric mode (flag bit 0), counted
    over the flag bits of the packed K and V caches."""
    import torch
    pop = torch.tensor([bin(i).count("1") for i in range(256)], dtype=torch.int64,
                       device=caches_kv[0].device)
    out = {}
    for name, t in zip(("K", "V"), caches_kv):
        f = t.view(rows, nb, fmt.block_bytes)[:, :, fmt.flag_offset:fmt.flag_offset + fmt.flag_bytes]
        ones = int(pop[f.reshape(-1).long()].sum())
        groups = rows * nb * 128 * 4
        out[name] = round(1.0 - ones / groups, 5)
    out["all"] = round((out["K"] + out["V"]) / 2, 5)
    return out


def warm_clocks(dev, n=1000):
    """~100 ms of device copies (256 MB each): the GPU reaches steady clocks only after tens
    of milliseconds of load."""
    import torch
    big = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    for _ in range(n):
        big2.copy_(big)
    torch.cuda.synchronize()
    del big, big2


def config_bench(name, args, K, S, dev, sptr, timed, cu):
    """Step (decode + combine) and back-to-back decode of one more workload, with the same
    rotation over cache copies as the headline figure."""
    import numpy as np
    import torch
    wl = S.WORKLOADS[name]
    fmt = K.Format(wl.bits, 128, wl.hybrid)
    rows, bb, nb = wl.B * wl.Hkv, fmt.block_bytes, wl.n_packed // 128
    S_ = K.suggest_splits(wl.B, wl.Hkv, wl.L, cu)
    x = S.make_inputs(wl)
    kps, vps = x.packed_src()
    kr, vr = x.residual()
    kp0 = torch.empty((rows, nb * bb), dtype=torch.uint8, device=dev)
    vp0 = torch.empty_like(kp0)
    for src, dst in ((kps, kp0), (vps, vp0)):
        sd = torch.from_numpy(np.ascontiguousarray(src.reshape(rows, wl.n_packed, 128))).to(dev)
        K.kvq_quantize_pack(fmt, sd, rows, wl.n_packed, wl.n_packed * 128, 128, dst, nb * bb, 0)
        del sd
    del kps, vps
    step_bytes = wl.step_bytes()
    copies = max(2, math.ceil(2 * MALL_BYTES / step_bytes) + 1)
    kr_d, vr_d = torch.from_numpy(kr).to(dev), torch.from_numpy(vr).to(dev)
    caches = [(kp0, vp0, kr_d, vr_d)] + [(kp0.clone(), vp0.clone(), kr_d.clone(), vr_d.clone())
                                         for _ in range(copies - 1)]
    q = torch.from_numpy(x.q).to(dev)
    po = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=dev)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device=dev)
    sm = float(np.float32(1.0 / math.sqrt(128)))

    def decode(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed, krd, vrd,
                               128, wl.n_res, sm, S_, po, pl, stream=sp)

    def step(i, sp=sptr):
        decode(i, sp)
        K.kvq_combine(po, pl, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    wsn = K.kvq_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, S_)
    ws = torch.zeros(max(wsn, 256), dtype=torch.uint8, device=dev)

    def fused(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention_fused(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed,
                                     krd, vrd, 128, wl.n_res, sm, S_, ws, ws.numel(), out,
                                     K.KVQ_OUT_F16, stream=sp)

    n = args.per_config_steps
    warm_clocks(dev)        # the GPU idled while the inputs were generated on the host
    # three interleaved rounds, each loop behind its own warm-up; the median of the rounds
    # (the clock drifts by a few percent over a long run)
    import statistics
    meas = {"step": [], "dec": [], "fused": []}
    for _ in range(3):
        meas["step"].append(timed(step, n, 100))
        meas["dec"].append(timed(decode, n, 50))
        meas["fused"].append(timed(fused, n, 50))
    step_ms, dec_ms, fused_ms = (statistics.median(meas[k]) for k in ("step", "dec", "fused"))
    res = {"B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "L": wl.L, "bits": wl.bits,
           "hybrid": wl.hybrid, "splits": S_, "cache_copies": copies,
           "algorithmic_bytes_per_step": step_bytes,
           "us_per_step": round(step_ms * 1e3, 3),
           "decode_kernel_us": round(dec_ms * 1e3, 3),
           "us_per_step_fused": round(fused_ms * 1e3, 3),
           "GB_per_s_step": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
           "GB_per_s_decode": round(step_bytes / (dec_ms * 1e-3) / 1e9, 1),
           "frac_step": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "frac_decode": round(step_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if wl.hybrid:
        res["sym_mode_share"] = flag_sym_ratio(fmt, (kp0, vp0), rows, nb)
    if wl.n_res == 128:
        # a decode step with one appended token (folded into the decode) and the flush of
        # the full window every 128 steps: quantize 128 tokens of every row, K and V
        fdst = torch.empty((rows, bb), dtype=torch.uint8, device=dev)

        def flush(i, sp=sptr):
            _, _, krd, vrd = caches[i % copies]
            K.kvq_quantize_pack(fmt, krd, rows, 128, 128 * 128, 128, fdst, bb, 0, stream=sp)
            K.kvq_quantize_pack(fmt, vrd, rows, 128, 128 * 128, 128, fdst, bb, 0, stream=sp)

        kn = torch.zeros((wl.B, wl.Hkv, 128), dtype=torch.float16, device=dev)

        def serve(i, sp=sptr):
            kp, vp, krd, vrd = caches[i % copies]
            K.kvq_decode_attention_append(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb,
                                          wl.n_packed, krd, vrd, 128, wl.n_res, kn, kn, sm, S_,
                                          po, pl, stream=sp)
            K.kvq_combine(po, pl, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

        fl_ms = timed(flush, 50, 5)
        sv_ms = timed(serve, n, 5)
        res["flush_us"] = round(fl_ms * 1e3, 3)
        res["append_decode_combine_us"] = round(sv_ms * 1e3, 3)
        res["step_us_with_append_and_amortized_flush"] = round((sv_ms + fl_ms / 128) * 1e3, 3)
    del caches, kp0, vp0, kr_d, vr_d
    torch.cuda.empty_cache()
    return res


def stream_read_reference(K, caches, copies, step_bytes, sink, sptr, timed):
    """The plain streaming read (kvq_stream_read) of one cache copy's bytes per launch, over
    the same rotation as the decode: the read ceiling of this memory system for the step's
    bytes."""
    def rd(i, sp=sptr):
        K.kvq_stream_read(list(caches[i % copies]), sink, stream=sp)
    ms = timed(rd, 500, 20)
    return {"bytes": step_bytes, "us": round(ms * 1e3, 3),
            "GB_per_s": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def paged_bench(args, K, S, dev, stream, sptr, timed):
    import numpy as np
    import torch
    pw = S.PAGED_WORKLOADS[args.paged_workload]
    x = S.make_paged_inputs(pw)
    fmt = K.Format(pw.bits, 128, pw.hybrid)
    bb = fmt.block_bytes
    B, Hkv, Hq, cap = pw.B, pw.Hkv, pw.Hq, pw.res_cap
    # one spare block per sequence after its last one, so the timed steps (each appends a
    # token to every sequence and evicts one into the packed cache) always have room
    maxb = x.table.shape[1] + 1
    tbl_np = np.full((B, maxb), -1, np.int32)
    tbl_np[:, :maxb - 1] = x.table
    for b in range(B):
        tbl_np[b, (int(x.n_packed[b]) + 127) // 128] = x.n_pool_blocks + b
    npool = x.n_pool_blocks + B
    bs, hs = Hkv * bb, bb
    tbl = torch.from_numpy(tbl_np).to(dev)
    # packed cache built on the GPU, one sequence at a time
    kpool = torch.zeros((npool, Hkv, bb), dtype=torch.uint8, device=dev)
    vpool = torch.zeros_like(kpool)
    for b in range(B):
        n = int(x.n_packed[b])
        if n == 0:
            continue
        cnt = torch.tensor([n], dtype=torch.int32, device=dev)
        zero = torch.zeros(1, dtype=torch.int32, device=dev)
        for src, pool in ((x.k_src[b], kpool), (x.v_src[b], vpool)):
            sd = torch.from_numpy(np.ascontiguousarray(src)).to(dev)
            K.kvq_pack_tokens_paged(fmt, sd, 1, Hkv, n * 128, 128, cnt, zero, n, pool, npool,
                                    bs, hs, tbl[b:b + 1], maxb)
            del sd
    step_bytes = x.step_bytes()
    copies = max(2, math.ceil(2 * MALL_BYTES / step_bytes) + 1)
    kr0 = torch.from_numpy(x.k_res).to(dev)
    vr0 = torch.from_numpy(x.v_res).to(dev)
    st0 = np.zeros((B, 4), np.int32)
    st0[:, 0], st0[:, 1], st0[:, 2] = x.n_packed, x.n_res, 0
    state0 = torch.from_numpy(st0).to(dev)
    st_init = state0.clone()
    caches = [(kpool, vpool, kr0, vr0, state0)] + [
        (kpool.clone(), vpool.clone(), kr0.clone(), vr0.clone(), state0.clone())
        for _ in range(copies - 1)]
    q = torch.from_numpy(x.q).to(dev)
    S_ = args.paged_splits or K.suggest_splits_paged(
        int(x.n_packed.sum()), int(x.n_packed.max()), Hkv,
        torch.cuda.get_device_properties(dev).multi_processor_count)
    po = torch.empty((B, Hq, S_, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((B, Hq, S_), dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    kn = torch.zeros((B, Hkv, 128), dtype=torch.float16, device=dev)
    sm = float(np.float32(1.0 / math.sqrt(128)))

    def decode(i, sp=sptr):
        kp, vp, krd, vrd, st = caches[i % copies]
        K.kvq_decode_attention_paged(fmt, q, B, Hq, Hkv, kp, vp, npool, bs, hs, tbl, maxb, st,
                                     krd, vrd, cap, sm, S_, po, pl, stream=sp)

    def update(i, sp=sptr):
        kp, vp, krd, vrd, st = caches[i % copies]
        K.kvq_append_evict(fmt, kn, kn, krd, vrd, cap, 0, kp, vp, npool, bs, hs, tbl, maxb, st,
                           B, Hkv, stream=sp)

    def step_separate(i, sp=sptr):
        update(i, sp)
        decode(i, sp)
        K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    # the folded step: kvq_decode_attention_paged_append applies the update inside the
    # decode; it reads a state buffer and writes the next one, so every copy keeps two and
    # alternates between them
    alt = [st.clone() for (_, _, _, _, st) in caches]
    cur = [0] * copies

    def fold(i, sp=sptr):
        c = i % copies
        kp, vp, krd, vrd, st = caches[c]
        s_in, s_out = (st, alt[c]) if cur[c] == 0 else (alt[c], st)
        K.kvq_decode_attention_paged_append(fmt, q, B, Hq, Hkv, kp, vp, npool, bs, hs, tbl, maxb,
                                            s_in, s_out, krd, vrd, cap, 0, kn, kn, sm, S_, po,
                                            pl, stream=sp)
        cur[c] ^= 1

    def combine(i, sp=sptr):
        K.kvq_combine(po, pl, B, Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    def step(i, sp=sptr):
        fold(i, sp)
        combine(i, sp)

    # one step both ways from the same cache (copies 0 and 1 are equal before any step):
    # partials, pools, windows and states must agree bit for bit
    step_separate(0)
    po_s, pl_s = po.clone(), pl.clone()
    step(1)
    torch.cuda.synchronize()
    a, b_ = caches[0], caches[1]
    identical = bool(torch.equal(po_s, po) and torch.equal(pl_s, pl) and
                     all(torch.equal(u, v) for u, v in zip(a[:4], b_[:4])) and
                     torch.equal(a[4], alt[1]))
    del po_s, pl_s

    wsb = K.kvq_decode_workspace_bytes(B, Hq, Hkv, S_)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def decode_fused(i, sp=sptr):
        kp, vp, krd, vrd, st = caches[i % copies]
        K.kvq_decode_attention_paged_fused(fmt, q, B, Hq, Hkv, kp, vp, npool, bs, hs, tbl, maxb,
                                           st, krd, vrd, cap, sm, S_, ws, wsb, out,
                                           K.KVQ_OUT_F16, stream=sp)

    def reset():
        # every copy back to the starting lengths (the pool and window bytes an update
        # wrote stay; the next updates write the same positions again)
        for c in range(copies):
            caches[c][4].copy_(st_init)
            alt[c].copy_(st_init)
            cur[c] = 0

    # every sequence grows by one packed token per update and its spare block holds 128:
    # the states are reset before each timed loop that updates. The loops run in rounds,
    # interleaved, and each figure is the median over the rounds (the clock drifts by a
    # few percent over a run).
    n = min(args.steps, 40)
    meas = {k: [] for k in ("step", "sep", "fold", "dec", "comb", "decf", "upd")}
    for _ in range(5):
        reset()
        meas["dec"].append(timed(decode, n, 3))
        meas["fold"].append(timed(fold, n, 2))
        reset()
        meas["step"].append(timed(step, n, 2))
        reset()
        meas["sep"].append(timed(step_separate, n, 2))
        reset()
        meas["upd"].append(timed(update, n, 2))
        meas["comb"].append(timed(combine, n, 3))
        meas["decf"].append(timed(decode_fused, n, 3))
    med = {k: float(np.median(v)) for k, v in meas.items()}
    step_ms, sep_ms, fold_ms, dec_ms = med["step"], med["sep"], med["fold"], med["dec"]
    comb_ms, decf_ms, upd_ms = med["comb"], med["decf"], med["upd"]
    res = {"workload": pw.name, "B": B, "Hq": Hq, "Hkv": Hkv, "bits": pw.bits,
           "lengths": [int(v) for v in (x.n_packed + x.n_res)], "splits": S_,
           "cache_copies": copies, "step_bytes": step_bytes,
           "us_per_step": round(step_ms * 1e3, 3),
           "us_per_step_separate_update": round(sep_ms * 1e3, 3),
           "folded_step_bit_identical": identical,
           "decode_kernel_us": round(dec_ms * 1e3, 3),
           "decode_append_kernel_us": round(fold_ms * 1e3, 3),
           "combine_us": round(comb_ms * 1e3, 3),
           "decode_fused_us": round(decf_ms * 1e3, 3),
           "append_evict_us": round(upd_ms * 1e3, 3),
           "GB_per_s_step": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
           "GB_per_s_decode": round(step_bytes / (dec_ms * 1e-3) / 1e9, 1),
           "frac_decode": round(step_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del caches, kpool, vpool
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth_inputs as S
    from bit_kv_cache_pack_amd import kvq as K

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = S.WORKLOADS[args.workload]
    fmt = K.Format(wl.bits, 128, wl.hybrid)
    rows = wl.B * wl.Hkv
    bb = fmt.block_bytes
    nb = wl.n_packed // 128
    S_ = args.splits or K.suggest_splits(wl.B, wl.Hkv, wl.L,
                                         torch.cuda.get_device_properties(dev).multi_processor_count)
    sm = float(np.float32(1.0 / math.sqrt(128)))

    x = S.make_inputs(wl)
    kps, vps = x.packed_src()
    kr, vr = x.residual()
    kps_d = torch.from_numpy(np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))).to(dev)
    vps_d = torch.from_numpy(np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))).to(dev)
    kp0 = torch.empty((rows, nb * bb), dtype=torch.uint8, device=dev)
    vp0 = torch.empty_like(kp0)
    K.kvq_quantize_pack(fmt, kps_d, rows, wl.n_packed, wl.n_packed * 128, 128, kp0, nb * bb, 0)
    K.kvq_quantize_pack(fmt, vps_d, rows, wl.n_packed, wl.n_packed * 128, 128, vp0, nb * bb, 0)
    del vps_d
    step_bytes = wl.step_bytes()
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / step_bytes) + 1)
    kr_d = torch.from_numpy(kr).to(dev)
    vr_d = torch.from_numpy(vr).to(dev)
    caches = [(kp0, vp0, kr_d, vr_d)] + [(kp0.clone(), vp0.clone(), kr_d.clone(), vr_d.clone())
                                         for _ in range(copies - 1)]
    q = torch.from_numpy(x.q).to(dev)
    part_o = torch.empty((wl.B, wl.Hq, S_, 128), dtype=torch.float32, device=dev)
    part_lse = torch.empty((wl.B, wl.Hq, S_), dtype=torch.float32, device=dev)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def decode(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed, krd, vrd,
                               128, wl.n_res, sm, S_, part_o, part_lse, stream=sp)

    def decode_valu(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention_valu(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed,
                                    krd, vrd, 128, wl.n_res, sm, S_, part_o, part_lse, stream=sp)

    def step(i, sp=sptr):
        decode(i, sp)
        K.kvq_combine(part_o, part_lse, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(n):
            fn(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / n

    # plain device copy as a bandwidth reference (read + write bytes). It runs before every
    # timed loop and for ~100 ms (1000 copies of 256 MB): the GPU reaches steady clocks only
    # after tens of milliseconds of load, so the copies also bring it there.
    big = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    for _ in range(1000):
        big2.copy_(big)
    t_start.record(stream)
    for _ in range(10):
        big2.copy_(big)
    t_end.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * big.numel() * 10 / (t_start.elapsed_time(t_end) * 1e-3) / 1e9
    del big, big2

    # W untimed warm-up steps, then exactly K timed steps back to back (the host enqueues
    # faster than the GPU runs them, so the GPU is never idle waiting for a launch)
    ms_per_step = timed(step, args.steps, args.warmup)
    # decode kernel duration: K launches back to back on the launch stream, between two HIP
    # events (an upper bound on the kernel's own duration: it includes the gaps between
    # launches). This is the figure the roofline uses.
    dec_ms = timed(decode, args.steps, 5)
    # the VALU-only comparison kernel (same partials, no matrix cores), timed the same way
    valu_ms = timed(decode_valu, args.steps, 5)
    # the same step as one launch: the splits merged inside the decode launch
    # (kvq_decode_attention_fused, caller-owned workspace)
    wsn = K.kvq_decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, S_)
    ws = torch.zeros(max(wsn, 256), dtype=torch.uint8, device=dev)

    def fused(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention_fused(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed,
                                     krd, vrd, 128, wl.n_res, sm, S_, ws, ws.numel(), out,
                                     K.KVQ_OUT_F16, stream=sp)

    fused_ms = timed(fused, args.steps, 5)
    # the read ceiling: a plain streaming read of the same bytes, same rotation
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    stream_ref = stream_read_reference(K, caches, copies, step_bytes, sink, sptr, timed)
    # the same K steps replayed from a HIP graph captured once, for reference
    cap_stream = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        sp = torch.cuda.current_stream(dev).cuda_stream
        for i in range(args.steps):
            step(i, sp)
    g.replay()
    torch.cuda.synchronize()
    t_start.record(stream)
    g.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    graph_ms = t_start.elapsed_time(t_end) / args.steps
    del g

    # FP16 flash-decoding baseline over the same tokens, uncompressed (the comparison the
    # pages report their speed-ups against): kvq_decode_attention_fp16 + kvq_combine
    fp16 = None
    if not args.no_fp16_baseline:
        f16_bytes = rows * wl.L * 128 * 2 * 2
        copies_f = max(2, math.ceil(2 * MALL_BYTES / f16_bytes) + 1)
        kf0 = torch.from_numpy(np.ascontiguousarray(x.k.reshape(rows, wl.L, 128))).to(dev)
        vf0 = torch.from_numpy(np.ascontiguousarray(x.v.reshape(rows, wl.L, 128))).to(dev)
        fcaches = [(kf0, vf0)] + [(kf0.clone(), vf0.clone()) for _ in range(copies_f - 1)]
        S16 = K.suggest_splits(wl.B, wl.Hkv, wl.L, 128)     # one workgroup per CU (LDS)
        po16 = torch.empty((wl.B, wl.Hq, S16, 128), dtype=torch.float32, device=dev)
        pl16 = torch.empty((wl.B, wl.Hq, S16), dtype=torch.float32, device=dev)

        def dec16(i, sp=sptr):
            kf, vf = fcaches[i % copies_f]
            K.kvq_decode_attention_fp16(q, wl.B, wl.Hq, wl.Hkv, kf, vf, wl.L, wl.L, sm, S16, po16,
                                        pl16, stream=sp)

        def step16(i, sp=sptr):
            dec16(i, sp)
            K.kvq_combine(po16, pl16, wl.B, wl.Hq, 128, S16, out, K.KVQ_OUT_F16, stream=sp)

        f16_step_ms = timed(step16, args.steps, args.warmup)
        f16_dec_ms = timed(dec16, args.steps, 5)
        fp16 = {"splits": S16, "cache_copies": copies_f, "bytes_per_step": f16_bytes,
                "us_per_step": round(f16_step_ms * 1e3, 3),
                "decode_kernel_us": round(f16_dec_ms * 1e3, 3),
                "GB_per_s_step": round(f16_bytes / (f16_step_ms * 1e-3) / 1e9, 2),
                "speedup_of_packed_step": round(f16_step_ms / ms_per_step, 3),
                "speedup_of_packed_decode_kernel": round(f16_dec_ms / dec_ms, 3)}
        del fcaches, kf0, vf0

    # the outer-dimension (KIVI-style) grouping over the same tokens, same bytes per step:
    # kvq_decode_attention_outer + kvq_combine, the comparison the InnerQ page draws
    outer = None
    if not args.no_outer and not wl.hybrid:
        ocaches = []
        for c in range(copies):
            ko = torch.empty_like(kp0)
            vo = torch.empty_like(vp0)
            ocaches.append((ko, vo, caches[c][2], caches[c][3]))
        ks_d = torch.from_numpy(np.ascontiguousarray(kps.reshape(rows, wl.n_packed, 128))).to(dev)
        vs_d = torch.from_numpy(np.ascontiguousarray(vps.reshape(rows, wl.n_packed, 128))).to(dev)
        for ko, vo, _, _ in ocaches:
            K.kvq_quantize_pack_outer(fmt, ks_d, rows, wl.n_packed, wl.n_packed * 128, 128, ko,
                                      nb * bb, 0)
            K.kvq_quantize_pack_outer(fmt, vs_d, rows, wl.n_packed, wl.n_packed * 128, 128, vo,
                                      nb * bb, 0)
        del ks_d, vs_d

        def decode_o(i, sp=sptr):
            kp, vp, krd, vrd = ocaches[i % copies]
            K.kvq_decode_attention_outer(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb,
                                         wl.n_packed, krd, vrd, 128, wl.n_res, sm, S_, part_o,
                                         part_lse, stream=sp)

        def step_o(i, sp=sptr):
            decode_o(i, sp)
            K.kvq_combine(part_o, part_lse, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

        o_step_ms = timed(step_o, args.steps, args.warmup)
        o_dec_ms = timed(decode_o, args.steps, 5)
        outer = {"us_per_step": round(o_step_ms * 1e3, 3),
                 "decode_kernel_us": round(o_dec_ms * 1e3, 3),
                 "GB_per_s_step": round(step_bytes / (o_step_ms * 1e-3) / 1e9, 1),
                 "inner_speedup_step": round(o_step_ms / ms_per_step, 3),
                 "inner_speedup_decode_kernel": round(o_dec_ms / dec_ms, 3)}
        if fp16 is not None:
            outer["speedup_over_fp16_step"] = round(fp16["us_per_step"] / (o_step_ms * 1e3), 3)
        del ocaches

    # key-channel normalization: the once-per-prefill passes over the fp16 prefill keys
    # (kvq_key_norm: 2 B read per element; kvq_channel_scale: 2 B read + 2 B written), and
    # the decode step with q scaled inside the decode kernel (kvq_decode_attention_knorm)
    knorm = None
    if not args.no_key_norm:
        kbytes = rows * wl.n_packed * 128 * 2
        copies_k = max(2, math.ceil(2 * MALL_BYTES / kbytes) + 1)
        ksrc = [kps_d] + [kps_d.clone() for _ in range(copies_k - 1)]
        kdst = [torch.empty_like(kps_d) for _ in range(copies_k)]
        nd = torch.empty((rows, 128), dtype=torch.float32, device=dev)
        K.kvq_key_norm(kps_d, rows, wl.n_packed, wl.n_packed * 128, 128, 128, nd)

        def key_norm(i, sp=sptr):
            K.kvq_key_norm(ksrc[i % copies_k], rows, wl.n_packed, wl.n_packed * 128, 128, 128,
                           nd, stream=sp)

        def key_scale(i, sp=sptr):
            K.kvq_channel_scale(ksrc[i % copies_k], rows, wl.n_packed, wl.n_packed * 128, 128,
                                128, nd, 1, K.KVQ_SCALE_DIVIDE, kdst[i % copies_k],
                                wl.n_packed * 128, 128, stream=sp)

        def decode_kn(i, sp=sptr):
            kp, vp, krd, vrd = caches[i % copies]
            K.kvq_decode_attention_knorm(fmt, q, nd, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb,
                                         wl.n_packed, krd, vrd, 128, wl.n_res, sm, S_, part_o,
                                         part_lse, stream=sp)

        def step_kn(i, sp=sptr):
            decode_kn(i, sp)
            K.kvq_combine(part_o, part_lse, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

        reps = 50
        kn_ms = timed(key_norm, reps, 3)
        ks_ms = timed(key_scale, reps, 3)
        step_kn_ms = timed(step_kn, args.steps, args.warmup)
        dec_kn_ms = timed(decode_kn, args.steps, 5)
        knorm = {"prefill_tokens": wl.n_packed, "key_bytes": kbytes, "copies": copies_k,
                 "key_norm_us": round(kn_ms * 1e3, 3),
                 "key_norm_GB_per_s": round(kbytes / (kn_ms * 1e-3) / 1e9, 1),
                 "channel_scale_keys_us": round(ks_ms * 1e3, 3),
                 "channel_scale_GB_per_s": round(2 * kbytes / (ks_ms * 1e-3) / 1e9, 1),
                 "step_knorm_us": round(step_kn_ms * 1e3, 3),
                 "decode_kernel_knorm_us": round(dec_kn_ms * 1e3, 3)}
        del ksrc, kdst
    del kps_d

    # paged cache: a serving-shaped batch of ragged sequences whose blocks are scattered
    # over one pool. One step = kvq_decode_attention_paged_append (the new token of every
    # sequence enters its window, evicting the oldest recent token into the packed cache,
    # inside the decode launch) + kvq_combine; the same step as three calls
    # (kvq_append_evict, kvq_decode_attention_paged, kvq_combine) is reported beside it.
    # Bytes = the step's algorithmic decode bytes.
    paged = None
    if not args.no_paged:
        paged = paged_bench(args, K, S, dev, stream, sptr, timed)

    # flush (quantize the full 128-token window of every row, K and V) and append
    fl_reps = 50
    fsrc = [(c[2], c[3]) for c in caches]
    fdst = torch.empty((rows, bb), dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(fl_reps + 5):
        if i == 5:
            e0.record(stream)
        kr_, vr_ = fsrc[i % copies]
        K.kvq_quantize_pack(fmt, kr_, rows, 128, 128 * 128, 128, fdst, bb, 0, stream=sptr)
        K.kvq_quantize_pack(fmt, vr_, rows, 128, 128 * 128, 128, fdst, bb, 0, stream=sptr)
    e1.record(stream)
    torch.cuda.synchronize()
    flush_ms = e0.elapsed_time(e1) / fl_reps
    kn = torch.zeros((wl.B, wl.Hkv, 128), dtype=torch.float16, device=dev)
    scratch_res = [torch.empty_like(kr_d), torch.empty_like(vr_d)]
    for i in range(fl_reps + 5):
        if i == 5:
            e0.record(stream)
        K.kvq_append_residual(kn, kn, scratch_res[0], scratch_res[1], wl.B, wl.Hkv, 128, 128,
                              i % 128, stream=sptr)
    e1.record(stream)
    torch.cuda.synchronize()
    append_ms = e0.elapsed_time(e1) / fl_reps

    # a serving step: the new token into window slot n_res - 1, the decode, the combine; as
    # three calls, and with the append folded into the decode (kvq_decode_attention_append)
    def serve3(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_append_residual(kn, kn, krd, vrd, wl.B, wl.Hkv, 128, 128, wl.n_res - 1, stream=sp)
        decode(i, sp)
        K.kvq_combine(part_o, part_lse, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    def serve2(i, sp=sptr):
        kp, vp, krd, vrd = caches[i % copies]
        K.kvq_decode_attention_append(fmt, q, wl.B, wl.Hq, wl.Hkv, kp, vp, nb * bb, wl.n_packed,
                                      krd, vrd, 128, wl.n_res, kn, kn, sm, S_, part_o, part_lse,
                                      stream=sp)
        K.kvq_combine(part_o, part_lse, wl.B, wl.Hq, 128, S_, out, K.KVQ_OUT_F16, stream=sp)

    serve = None
    if wl.n_res >= 1:
        serve3_ms = timed(serve3, args.steps, 5)
        serve2_ms = timed(serve2, args.steps, 5)
        serve = {"append_decode_combine_us": round(serve3_ms * 1e3, 3),
                 "fused_append_decode_combine_us": round(serve2_ms * 1e3, 3)}

    # the same K steps timed once more, after every other headline measurement: a clock
    # still ramping up during the first timed loop would show as a lower figure here
    repeat_ms = timed(step, args.steps, 5)

    per_config = None
    if not args.no_per_config:
        del caches
        torch.cuda.empty_cache()
        cu = torch.cuda.get_device_properties(dev).multi_processor_count
        per_config = {n: config_bench(n, args, K, S, dev, sptr, timed, cu)
                      for n in ("tiny", "batch8_2bit_hybrid", "long_128k_3bit", "mha_b64_append")
                      if n != wl.name}

    achieved = step_bytes / (dec_ms * 1e-3) / 1e9
    traffic = recorded_traffic(wl.name)
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "decode_kernel_us": round(dec_ms * 1e3, 3),
        "us_per_step_graph_replay": round(graph_ms * 1e3, 3),
        "us_per_step_repeat": round(repeat_ms * 1e3, 3),
        "us_per_step_fused": round(fused_ms * 1e3, 3),
        "decode_kernel_valu_only_us": round(valu_ms * 1e3, 3),
        "flush_us": round(flush_ms * 1e3, 3),
        "append_us": round(append_ms * 1e3, 3),
        "step_us_with_append_and_amortized_flush": round((ms_per_step + append_ms + flush_ms / 128)
                                                         * 1e3, 3),
        "serving_step": serve,
        "copy_reference_gbps": round(copy_gbps, 1),
        "stream_read_reference": dict(stream_ref, decode_over_read_time=round(
            dec_ms * 1e3 / stream_ref["us"], 3)),
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "L": wl.L,
                   "bits": wl.bits, "group": 32, "hybrid": wl.hybrid, "n_packed": wl.n_packed,
                   "n_res": wl.n_res, "splits": S_, "cache_copies": copies,
                   "algorithmic_bytes_per_step": step_bytes},
        "fp16_baseline": fp16,
        "key_norm": knorm,
        "outer_grouping": outer,
        "paged": paged,
        "per_config": per_config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "decode_kernel (kvq_decode_attention)"},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds, args.cpu_single_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
