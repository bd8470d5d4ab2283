"""Pins for the oracle's weight_sumsq, the ||W||_F^2 that the normalized
update ([RGC], "How it works") scales by and that a carried-norm update hands
to the next step (CPU only).

Checked against closed forms: a constant matrix (d k c^2), one nonzero entry,
exact scaling by powers of two, a sum of squares of known integers, and the
normalized update's own reported ||W||.
"""
import numpy as np

import oracle as orc


def _bf16(vals):
    return orc.f32_to_bf16_rne(np.asarray(vals, dtype=np.float32))


def test_constant_matrix():
    for d, k, c in ((4, 8, 0.5), (16, 24, -3.0), (7, 5, 0.015625)):
        w = _bf16(np.full((d, k), c))
        assert orc.weight_sumsq(w) == d * k * c * c


def test_single_entry_and_zero():
    w = _bf16(np.zeros((6, 9)))
    assert orc.weight_sumsq(w) == 0.0
    w = _bf16(np.where(np.arange(54).reshape(6, 9) == 31, -1.25, 0.0))
    assert orc.weight_sumsq(w) == 1.5625


def test_integers():
    # bf16 holds the integers -256..256 exactly; sum of i^2 for i = 1..n is n(n+1)(2n+1)/6
    n = 200
    w = _bf16(np.arange(1, n + 1, dtype=np.float32).reshape(8, 25))
    assert orc.weight_sumsq(w) == n * (n + 1) * (2 * n + 1) / 6
    assert orc.weight_sumsq(_bf16(-np.arange(1, n + 1, dtype=np.float32).reshape(8, 25))) == \
        n * (n + 1) * (2 * n + 1) / 6


def test_power_of_two_scaling():
    rng = np.random.default_rng(3)
    w = _bf16(0.02 * rng.standard_normal((32, 48)))
    w4 = _bf16(4.0 * orc.bf16_to_f64(w))  # exact: a power of two times a bf16 value
    assert orc.weight_sumsq(w4) == 16.0 * orc.weight_sumsq(w)


def test_matches_update_stats():
    rng = np.random.default_rng(5)
    d, k, r = 8, 16, 4
    w = _bf16(0.02 * rng.standard_normal((d, k)))
    c = (rng.standard_normal((d, r)) * 0.1).astype(np.float32)
    p = orc.rademacher_projection(9, k, r)
    _, stats = orc.apply_update(w, c, p, 1e-3, 4)
    assert np.float32(np.sqrt(orc.weight_sumsq(w))) == stats[0]
