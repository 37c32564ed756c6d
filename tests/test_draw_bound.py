"""The rounding bound behind the pruning of sampled unconstrained rows.

The row kernel ranks a sampled candidate by
    r = fl(fl(c / pen) + g),  c = fl(S + fl(fl(x * it) - lse))
(all fp32, it = 1/T) and, while streaming the row before lse is known, bounds
it with the estimate y = fl(fl(x * q) + g), q = fl(it / pen).  Its pruning is
sound when, for every finite candidate,
    |r - (D + y)| <= 2^-20 (|y| + 32 + M),
    D = (S - lse) / pen,  M = (|S| + |lse|) / pen   (exact reals),
given |g| < 23 (the Gumbel variate of a word u = (r + 1/2) 2^-32 lies in
(-3.12, 22.9)).  Here the inequality is checked in IEEE fp32 arithmetic on
random and extreme operands; the error of the fast draw estimates, the
other term of the kernel's margin, is measured on the GPU over all 2^32
words (test_gpu_parity.test_draw_error_bound)."""
import math

import numpy as np

f32 = np.float32


def rank_and_estimate(x, it, S, lse, pen, g):
    with np.errstate(over="ignore", invalid="ignore"):
        c = f32(f32(S) + f32(f32(f32(x) * f32(it)) - f32(lse)))
        r = f32(f32(c / f32(pen)) + f32(g))
        q = f32(f32(it) / f32(pen))
        y = f32(f32(f32(x) * q) + f32(g))
    return c, r, y


def check(x, it, S, lse, pen, g):
    c, r, y = rank_and_estimate(x, it, S, lse, pen, g)
    if not (np.isfinite(c) and np.isfinite(r) and np.isfinite(y)):
        return None  # the kernel falls back to the exact path for such rows
    D = (float(S) - float(lse)) / float(pen)
    M = (abs(float(S)) + abs(float(lse))) / float(pen)
    err = abs(float(r) - (D + float(y)))
    bound = 2.0 ** -20 * (abs(float(y)) + 32.0 + M)
    return err, bound


def gumbel_range():
    lo = -math.log(-math.log(0.5 * 2.0 ** -32))
    hi = -math.log(-math.log(1.0 - 0.5 * 2.0 ** -32))
    return lo, hi


def test_gumbel_variates_lie_below_23():
    lo, hi = gumbel_range()
    assert -3.2 < lo < -3.1 and 22.8 < hi < 23.0


def test_random_operands_within_bound():
    rng = np.random.default_rng(7)
    lo, hi = gumbel_range()
    worst = 0.0
    for _ in range(60_000):
        scale = 10.0 ** rng.uniform(-3, 6)
        x = f32(rng.normal() * scale)
        it = f32(10.0 ** rng.uniform(-1.5, 1.5))
        S = f32(-abs(rng.normal()) * 10.0 ** rng.uniform(-2, 5))
        lse = f32(rng.normal() * 10.0 ** rng.uniform(-2, 6))
        pen = f32(10.0 ** rng.uniform(-0.5, 1.5)) if rng.random() < 0.5 else f32(1.0)
        g = f32(rng.uniform(lo, hi))
        res = check(x, it, S, lse, pen, g)
        if res is None:
            continue
        err, bound = res
        assert err <= bound, (x, it, S, lse, pen, g, err, bound)
        worst = max(worst, err / bound)
    assert worst < 0.5  # the margin carries at least a factor of two


def test_extreme_operands_within_bound():
    lo, hi = gumbel_range()
    big = [1e30, 3e37, 1.7e38]
    for x in [*big, *(-v for v in big), 0.0, 1e-40, -1e-40]:
        for it in (1.0, 0.5, 1.999, 0.01):
            for S in (0.0, -1e-3, -1e30, -1e37):
                for lse in (0.0, 1e37, -1e37, 12.5):
                    for pen in (1.0, 0.7, 9.0):
                        for g in (lo, 0.0, hi):
                            res = check(f32(x), f32(it), f32(S), f32(lse), f32(pen), f32(g))
                            if res is not None:
                                assert res[0] <= res[1], (x, it, S, lse, pen, g, res)


def test_bound_fails_without_its_terms():
    """The check can fail: with the |y| or M term dropped, large operands break it."""
    rng = np.random.default_rng(3)
    broke_y = broke_m = False
    for _ in range(20_000):
        x = f32(rng.normal() * 1e6)
        S = f32(-abs(rng.normal()) * 1e6)
        lse = f32(rng.normal() * 1e6)
        c, r, y = rank_and_estimate(x, f32(1.0), S, lse, f32(1.0), f32(0.5))
        D = float(S) - float(lse)
        err = abs(float(r) - (D + float(y)))
        M = abs(float(S)) + abs(float(lse))
        broke_y |= err > 2.0 ** -20 * (32.0 + M)
        broke_m |= err > 2.0 ** -20 * (abs(float(y)) + 32.0)
    assert broke_y or broke_m
