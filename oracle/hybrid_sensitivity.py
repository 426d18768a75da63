"""How often the hybrid quantizer's symmetric candidate wins, under the symmetric grid the
oracle uses and under two alternatives (test infrastructure: a CPU-only diagnostic).

The InnerQ page ("KV缓存量化技术InnerQ：提升大模型推理效率", sec. 2.2) has every group try
a symmetric and an asymmetric quantizer and keep the one with the lower error; its sec. 5
calls 30-70% of groups choosing the symmetric mode normal. The pages never define the
symmetric grid. The oracle's reading is the signed grid +-(2^(b-1) - 1) * s with
s = max|x| / (2^(b-1) - 1) (2-bit: three levels -s, 0, s). Two other plain readings:

  full   the full signed range -2^(b-1) .. 2^(b-1) - 1 of b-bit two's complement, with
         s = max|x| / 2^(b-1) when the largest magnitude is negative, else
         max|x| / (2^(b-1) - 1) (so every value is inside the grid);
  half   a grid symmetric about 0 with no zero level, (k + 1/2) * s for
         k = -2^(b-1) .. 2^(b-1) - 1, s = max|x| / (2^(b-1) - 1/2).

For each group the asymmetric candidate is the oracle's own (oq_asym_candidate, fp16 scale
and zero as stored); a symmetric candidate wins when its sum of squared errors is lower
(strictly, as in the oracle). The symmetric scales are rounded to fp16 like the stored
ones, codes are round-half-away-from-zero and clipped; errors are summed in fp64. The
"oracle" column is the share of flag-0 groups the oracle itself reports for the same
groups (binary32 errors in its pairwise order), a check that the fp64 re-evaluation of
the oracle's grid agrees.

    python -m oracle.hybrid_sensitivity [n_groups]
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402

G = 32


def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _round_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _sym_sse(x: np.ndarray, bits: int, kind: str) -> float:
    """SSE of one symmetric candidate for group x (float64 values of fp16 inputs)."""
    half = 1 << (bits - 1)
    m = float(np.max(np.abs(x)))
    if m == 0.0:
        return 0.0
    if kind == "oracle":
        lo, hi, offs = -(half - 1), half - 1, 0.0
        s = m / (half - 1)
    elif kind == "full":
        lo, hi, offs = -half, half - 1, 0.0
        neg_max = -float(np.min(x)) >= float(np.max(x))
        s = m / half if neg_max else m / (half - 1)
    elif kind == "half":
        lo, hi, offs = -half, half - 1, 0.5
        s = m / (half - 0.5)
    else:
        raise ValueError(kind)
    s = float(np.float16(s))
    if s == 0.0 or not np.isfinite(s):
        return float("inf")
    k = np.clip(_round_away(x / s - offs), lo, hi)
    return float(np.sum((x - (k + offs) * s) ** 2))


def _asym_sse(x16: np.ndarray, bits: int) -> float:
    a = O.asym_candidate(x16, bits)
    s = float(np.frombuffer(np.uint16(a.scale).tobytes(), np.float16)[0])
    z = float(np.frombuffer(np.uint16(a.zero).tobytes(), np.float16)[0])
    x = x16.astype(np.float64)
    return float(np.sum((x - (a.codes.astype(np.float64) * s + z)) ** 2))


def sym_shares(groups16: np.ndarray, bits: int) -> dict:
    """Share of groups whose symmetric candidate beats the asymmetric one, per grid."""
    wins = {"oracle": 0, "full": 0, "half": 0}
    flags0 = 0
    for g in groups16:
        x = g.astype(np.float64)
        ea = _asym_sse(g, bits)
        for kind in wins:
            if _sym_sse(x, bits, kind) < ea:
                wins[kind] += 1
        flags0 += O.quantize_group(g, bits, hybrid=True).flag == 0
    n = len(groups16)
    out = {k: v / n for k, v in wins.items()}
    out["oracle_flags"] = flags0 / n
    return out


def group_kinds(rng, n: int) -> dict:
    """Seeded groups of several value shapes (32 channels each)."""
    kinds = {
        "student_t5 (config-3 K/V)": rng.standard_t(5, size=(n, G)),
        "normal": rng.standard_normal((n, G)),
        "uniform [-1, 1]": rng.uniform(-1, 1, (n, G)),
        "uniform [0, 1] (one-signed)": rng.uniform(0, 1, (n, G)),
        "laplace": rng.laplace(size=(n, G)),
        "three levels {-a, 0, a} + 1% noise":
            rng.choice([-1.0, 0.0, 1.0], size=(n, G)) + 0.01 * rng.standard_normal((n, G)),
    }
    return {k: _f16(v) for k, v in kinds.items()}


def config3_groups(n: int) -> np.ndarray:
    """n groups from the batch8_2bit_hybrid recipe's K cache (first kv-head rows)."""
    import synth_inputs as S
    x = S.make_inputs(S.WORKLOADS["batch8_2bit_hybrid"], B=1, L=max(256, (n // 4) + 128))
    k = x.k.reshape(-1, 128)[: (n + 3) // 4]
    return np.ascontiguousarray(k.reshape(-1, G)[:n])


def main(n: int = 4000) -> None:
    rng = np.random.default_rng(7)
    rows = [("batch8_2bit_hybrid K (recipe)", config3_groups(n))]
    rows += list(group_kinds(rng, n).items())
    for bits in (2, 3, 4):
        print(f"{bits}-bit: share of groups picking the symmetric mode ({n} groups each)")
        print(f"  {'groups':40s} {'oracle grid':>12s} {'full range':>11s} {'half-int':>9s}"
              f" {'oracle flags':>13s}")
        for name, gs in rows:
            r = sym_shares(gs, bits)
            print(f"  {name:40s} {r['oracle']:12.4f} {r['full']:11.4f} {r['half']:9.4f}"
                  f" {r['oracle_flags']:13.4f}", flush=True)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 4000)
