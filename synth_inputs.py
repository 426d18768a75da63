"""Seeded synthetic inputs for the packed-KV decode path.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic (no quantization, no attention). Both the HIP path's tests/benchmark and the
CPU oracle take their inputs from here.

Recipe (one numpy PCG64 generator per workload, seed 0 unless stated): draw the
structure parameters first (outlier channels, per-head standard deviations), then K row
by row ([batch][kv-head] rows of [L][head_dim]), then V the same way, then q. fp32 draws
are cast to fp16 with round-to-nearest-even. Layout is [B][H][L][head_dim] with the
channels contiguous. The five workloads mirror the decode shapes the pages discuss
(LLaMA-3.1-8B 32K and 128K GQA decode on the BitDecoding page, batched 2-bit with sink and
recent windows on the InnerQ page, Llama-2-13B-sized batch decode on the Oaken page);
no dataset or trained weights are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
RES_CAP = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    bits: int
    hybrid: bool = False
    sink: int = 0                 # leading tokens kept in fp16 (slots 0..sink-1)
    dist: str = "normal"          # normal | student_t5 | normal_head_std
    outlier_channels: tuple = ()  # fixed K channels scaled by outlier_scale
    n_random_outliers: int = 0    # K channels picked with rng.choice(128, n, replace=False)
    outlier_scale: float = 1.0
    seed: int = 0
    description: str = ""
    res_cap: int = RES_CAP
    head_dim: int = HEAD_DIM

    @property
    def gq(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_res(self) -> int:
        return min(self.res_cap, self.L)

    @property
    def n_packed(self) -> int:
        return self.L - self.n_res

    def kv_bytes_per_token_head(self) -> int:
        """Algorithmic bytes read per (token, kv-head) for K+V from the packed cache."""
        ng = self.head_dim // 32
        return 2 * (self.head_dim * self.bits // 8 + ng * 4)

    def step_bytes(self, n_res: int | None = None) -> int:
        """Codes + fp16 scale/zero + fp16 residual bytes read by one decode step."""
        n_res = self.n_res if n_res is None else n_res
        rows = self.B * self.Hkv
        return rows * (self.n_packed * self.kv_bytes_per_token_head()
                       + n_res * 2 * self.head_dim * 2)


WORKLOADS = {
    "tiny": Workload(
        "tiny", B=1, Hq=8, Hkv=2, L=1024, bits=4, outlier_channels=(3, 77), outlier_scale=8.0,
        description="B1 8q/2kv L1024 4-bit asym, K ch 3,77 x8, 128 fp16 residual"),
    "llama8b_32k": Workload(
        "llama8b_32k", B=1, Hq=32, Hkv=8, L=32768, bits=4, n_random_outliers=4,
        outlier_scale=10.0,
        description="B1 32q/8kv L32768 4-bit asym, 4 random K ch x10, 128 fp16 residual"),
    "batch8_2bit_hybrid": Workload(
        "batch8_2bit_hybrid", B=8, Hq=32, Hkv=8, L=32768, bits=2, hybrid=True, sink=32,
        dist="student_t5",
        description="B8 32q/8kv L32768 2-bit hybrid sym/asym, Student-t(5) K,V, 32 sink + 96 recent"),
    "long_128k_3bit": Workload(
        "long_128k_3bit", B=1, Hq=32, Hkv=8, L=131072, bits=3, dist="normal_head_std",
        description="B1 32q/8kv L131072 3-bit asym, per-(K/V, kv-head) std ~ U[0.5,4]"),
    "mha_b64_append": Workload(
        "mha_b64_append", B=64, Hq=40, Hkv=40, L=4096, bits=4,
        description="B64 40q/40kv L4096 4-bit asym, 1 appended token per step, flush at 128"),
}


@dataclass
class Inputs:
    wl: Workload
    q: np.ndarray          # fp16 [B][Hq][d]
    k: np.ndarray          # fp16 [B][Hkv][L][d]
    v: np.ndarray
    rng: np.random.Generator = field(repr=False, default=None)
    meta: dict = field(default_factory=dict)

    def packed_src(self):
        """fp16 K, V of the tokens that go to the packed cache: [B][Hkv][n_packed][d]."""
        wl = self.wl
        lo, hi = wl.sink, wl.sink + wl.n_packed
        return self.k[:, :, lo:hi], self.v[:, :, lo:hi]

    def residual(self):
        """fp16 residual buffers [B][Hkv][res_cap][d]: sink tokens in slots 0..sink-1, the
        most recent tokens after them (slot order does not change the attention)."""
        wl = self.wl
        kr = np.zeros((wl.B, wl.Hkv, wl.res_cap, wl.head_dim), np.float16)
        vr = np.zeros_like(kr)
        s = wl.sink
        recent = wl.n_res - s
        kr[:, :, :s] = self.k[:, :, :s]
        vr[:, :, :s] = self.v[:, :, :s]
        kr[:, :, s:s + recent] = self.k[:, :, wl.L - recent:]
        vr[:, :, s:s + recent] = self.v[:, :, wl.L - recent:]
        return kr, vr


def _draw_rows(rng, B, H, L, d, dist, std=None, ch_mult=None):
    out = np.empty((B, H, L, d), np.float16)
    for b in range(B):
        for h in range(H):
            if dist == "student_t5":
                x = rng.standard_t(5, size=(L, d)).astype(np.float32)
            else:
                x = rng.standard_normal((L, d), dtype=np.float32)
                if std is not None:
                    x *= np.float32(std[h])
            if ch_mult is not None:
                x *= ch_mult
            out[b, h] = x.astype(np.float16)
    return out


def make_inputs(wl: Workload | str, seed: int | None = None, L: int | None = None,
                B: int | None = None) -> Inputs:
    """Draw q, K, V for a workload (optionally with a different L or B for small tests)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if L is not None or B is not None or seed is not None:
        kw = dict(wl.__dict__)
        if L is not None:
            kw["L"] = L
        if B is not None:
            kw["B"] = B
        if seed is not None:
            kw["seed"] = seed
        wl = Workload(**kw)
    rng = np.random.default_rng(wl.seed)
    d = wl.head_dim
    meta = {}
    ch = list(wl.outlier_channels)
    if wl.n_random_outliers:
        ch = sorted(int(c) for c in rng.choice(d, wl.n_random_outliers, replace=False))
    meta["outlier_channels"] = ch
    std_k = std_v = None
    if wl.dist == "normal_head_std":
        std_k = rng.uniform(0.5, 4.0, wl.Hkv).astype(np.float32)
        std_v = rng.uniform(0.5, 4.0, wl.Hkv).astype(np.float32)
        meta["std_k"], meta["std_v"] = std_k, std_v
    kdist = "student_t5" if wl.dist == "student_t5" else "normal"
    ch_mult = None
    if ch:
        ch_mult = np.ones(d, np.float32)
        ch_mult[ch] = np.float32(wl.outlier_scale)
    k = _draw_rows(rng, wl.B, wl.Hkv, wl.L, d, kdist, std_k, ch_mult)
    v = _draw_rows(rng, wl.B, wl.Hkv, wl.L, d, kdist, std_v)
    q = rng.standard_normal((wl.B, wl.Hq, d), dtype=np.float32).astype(np.float16)
    return Inputs(wl, q, k, v, rng, meta)


@dataclass(frozen=True)
class PagedWorkload:
    """Serving-shaped batch for the paged cache: B sequences of ragged lengths drawn
    uniformly from [L_min, L_max] (each sequence: min(L, res_cap) tokens in its fp16
    window, the rest packed), blocks of all sequences scattered over one pool."""
    name: str
    B: int
    Hq: int
    Hkv: int
    L_min: int
    L_max: int
    bits: int
    hybrid: bool = False
    res_cap: int = RES_CAP
    spare_blocks: int = 16        # pool blocks no sequence uses
    seed: int = 0
    description: str = ""
    head_dim: int = HEAD_DIM

    @property
    def gq(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes_per_token_head(self) -> int:
        ng = self.head_dim // 32
        return 2 * (self.head_dim * self.bits // 8 + ng * 4)


PAGED_WORKLOADS = {
    "paged_ragged_b16": PagedWorkload(
        "paged_ragged_b16", B=16, Hq=32, Hkv=8, L_min=1024, L_max=32768, bits=4,
        description="16 sequences, L ~ U[1K, 32K], 32q/8kv, 4-bit asym, 128-slot fp16 windows, "
                    "blocks scattered over one pool"),
}


@dataclass
class PagedInputs:
    wl: PagedWorkload
    q: np.ndarray               # fp16 [B][Hq][d]
    k_src: list                 # per sequence: fp16 [Hkv][n_packed_b][d] (packed part)
    v_src: list
    k_res: np.ndarray           # fp16 [B][Hkv][res_cap][d]
    v_res: np.ndarray
    n_packed: np.ndarray        # int32 [B]
    n_res: np.ndarray           # int32 [B]
    table: np.ndarray           # int32 [B][max_blocks], -1 where unused
    n_pool_blocks: int

    def step_bytes(self) -> int:
        """Codes + fp16 scale/zero of every packed token and the fp16 window tokens read by
        one decode step over the whole batch."""
        wl = self.wl
        return wl.Hkv * (int(self.n_packed.sum()) * wl.kv_bytes_per_token_head()
                         + int(self.n_res.sum()) * 2 * wl.head_dim * 2)


def make_paged_inputs(wl: PagedWorkload | str, seed: int | None = None) -> PagedInputs:
    """Lengths first, then per sequence K and V of its packed part and its window, then q,
    then the pool placement (a random permutation of the pool's blocks)."""
    if isinstance(wl, str):
        wl = PAGED_WORKLOADS[wl]
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    d = wl.head_dim
    L = rng.integers(wl.L_min, wl.L_max + 1, wl.B)
    n_res = np.minimum(L, wl.res_cap).astype(np.int32)
    n_packed = (L - n_res).astype(np.int32)
    k_src, v_src = [], []
    k_res = np.zeros((wl.B, wl.Hkv, wl.res_cap, d), np.float16)
    v_res = np.zeros_like(k_res)
    for b in range(wl.B):
        k_src.append(rng.standard_normal((wl.Hkv, int(n_packed[b]), d), dtype=np.float32)
                     .astype(np.float16))
        v_src.append(rng.standard_normal((wl.Hkv, int(n_packed[b]), d), dtype=np.float32)
                     .astype(np.float16))
        k_res[b, :, :n_res[b]] = rng.standard_normal((wl.Hkv, int(n_res[b]), d),
                                                     dtype=np.float32).astype(np.float16)
        v_res[b, :, :n_res[b]] = rng.standard_normal((wl.Hkv, int(n_res[b]), d),
                                                     dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((wl.B, wl.Hq, d), dtype=np.float32).astype(np.float16)
    nblk = [(int(n) + 127) // 128 for n in n_packed]
    n_pool = sum(nblk) + wl.spare_blocks
    perm = rng.permutation(n_pool)
    table = np.full((wl.B, max(max(nblk), 1)), -1, np.int32)
    k = 0
    for b, nb in enumerate(nblk):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    return PagedInputs(wl, q, k_src, v_src, k_res, v_res, n_packed, n_res, table, n_pool)


def append_step_inputs(rng: np.random.Generator, wl: Workload):
    """One decode step of the append workload: new K, V token per (batch, kv-head) and q."""
    d = wl.head_dim
    kn = rng.standard_normal((wl.B, wl.Hkv, d), dtype=np.float32).astype(np.float16)
    vn = rng.standard_normal((wl.B, wl.Hkv, d), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((wl.B, wl.Hq, d), dtype=np.float32).astype(np.float16)
    return kn, vn, q


def random_groups(rng: np.random.Generator, n: int, kind: str = "normal") -> np.ndarray:
    """n groups of 32 fp16 values with assorted shapes (used by quantizer property tests)."""
    if kind == "normal":
        x = rng.standard_normal((n, 32), dtype=np.float32)
    elif kind == "t5":
        x = rng.standard_t(5, size=(n, 32)).astype(np.float32)
    elif kind == "wide":
        x = rng.standard_normal((n, 32), dtype=np.float32) * np.float32(1000.0)
    elif kind == "tiny":
        x = rng.standard_normal((n, 32), dtype=np.float32) * np.float32(1e-6)
    elif kind == "offset":
        x = rng.standard_normal((n, 32), dtype=np.float32) + np.float32(50.0)
    elif kind == "few_levels":
        x = rng.integers(-3, 4, size=(n, 32)).astype(np.float32) * np.float32(0.25)
    elif kind == "ternary":
        a = rng.uniform(0.1, 10.0, size=(n, 1)).astype(np.float32)
        x = rng.integers(-1, 2, size=(n, 32)).astype(np.float32) * a
    else:
        raise ValueError(kind)
    return x.astype(np.float16)
