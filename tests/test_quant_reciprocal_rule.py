"""Host check of the rule the GPU quantizer uses to take a code from a reciprocal instead of
the correctly rounded division: with q = fl(d * r), r within one ulp of 1/s either way,
c = floor(fl(q + 1/2)) is accepted only when |q - c| < fl(1/2 - 2^-19 q), and an accepted c
must equal round_half_away(fl(d / s)), the code the quantizer's definition gives (fp32
throughout, as the kernel computes it). Inputs are fp16-derived like the kernel's: d = x -
zero of fp16 values, s an fp16 scale; many sit on or next to the rounding points."""
import numpy as np

f32 = np.float32


def _round_half_away_pos(t):
    k = np.trunc(t)
    return np.where(t - k >= f32(0.5), k + f32(1), k).astype(np.float32)


def _cases(rng, n, N):
    with np.errstate(over="ignore"):
        return _draw(rng, n, N)


def _draw(rng, n, N):
    s = (2.0 ** rng.uniform(-24, 12, n)).astype(np.float16).astype(np.float32)
    s = np.where(s == 0, f32(2.0 ** -24), s)
    z = np.where(rng.random(n) < 0.5, -(2.0 ** rng.uniform(-24, 10, n)),
                 2.0 ** rng.uniform(-24, -10, n)).astype(np.float16).astype(np.float32)
    k = rng.integers(0, N + 2, n)
    x = (z.astype(np.float64) + (k + 0.5) * s.astype(np.float64)).astype(np.float16)
    step = rng.integers(-3, 4, n)
    for j in range(3):
        x = np.where(step > j, np.nextafter(x, np.float16(np.inf)),
                     np.where(step < -j, np.nextafter(x, np.float16(-np.inf)), x))
    x = x.astype(np.float32)
    keep = np.isfinite(x) & (x >= z)
    d = (x[keep] - z[keep]).astype(np.float32)        # one fp32 subtraction, as the kernel
    return d, s[keep]


def test_reciprocal_rule_never_accepts_a_wrong_code():
    rng = np.random.default_rng(7)
    accepted = 0
    for N in (3, 7, 15):
        d, s = _cases(rng, 400_000, N)
        t = (d / s).astype(np.float32)                # correctly rounded fp32 quotient
        want = np.minimum(_round_half_away_pos(t), f32(N))
        r0 = (f32(1) / s).astype(np.float32)
        for r in (r0, np.nextafter(r0, f32(np.inf)), np.nextafter(r0, f32(0))):
            q = (d * r).astype(np.float32)
            c = np.floor((q + f32(0.5)).astype(np.float32)).astype(np.float32)
            thr = (0.5 - q.astype(np.float64) * 2.0 ** -19).astype(np.float32)   # one fma
            ok = np.abs((q - c).astype(np.float32)) < thr
            got = np.minimum(c, f32(N))
            bad = ok & (got != want)
            assert not bad.any(), (N, d[bad][:4], s[bad][:4])
            accepted += int(ok.sum())
        # the rule sends only a small share of elements to the exact division
        assert np.mean(~ok) < 0.5
    assert accepted > 1_000_000
