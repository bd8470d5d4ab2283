"""Pins for the oracle's fixed-step update W <- SR_bf16(W - alpha C P^T)
([LoGRA-M], "Minimal Causal Code": W -= alpha*eta*(U @ A), U = S, A = P^T)
(CPU only).

Checked against: brute force on a tiny matrix (explicit loops for H, the
pre-rounding value and both bf16 neighbours), the normalized update (the two
must agree when alpha is the normalized step), the identity at alpha = 0, and
the mean over rounding seeds.
"""
import numpy as np

import oracle as orc


def _tiny(seed=11, d=4, k=8, r=2):
    rng = np.random.default_rng(seed)
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    c = (rng.standard_normal((d, r)) * 0.5).astype(np.float32)
    p = orc.rademacher_projection(seed, k, r)
    return w, c, p


def test_brute_force_tiny_update():
    """Each output is the stochastic rounding of v_ij = w_ij - alpha * sum_a c_ia p_ja,
    formed with explicit loops (no matrix product), and lies on one of v's two
    bf16 neighbours."""
    w, c, p = _tiny()
    d, k = w.shape
    r = c.shape[1]
    alpha = np.float32(3e-3)
    got = orc.apply_scaled(w, c, p, alpha, seed=77)
    pv = orc.bf16_to_f64(p)
    wv = orc.bf16_to_f64(w)
    v = np.zeros((d, k), dtype=np.float32)
    for i in range(d):
        for j in range(k):
            h = 0.0
            for a in range(r):
                h += float(c[i, a]) * float(pv[j, a])
            v[i, j] = np.float32(np.float32(wv[i, j]) - np.float32(alpha * np.float32(h)))
    assert np.array_equal(got, orc.stochastic_round(v, orc.rounding_bits(77, d, k)))
    lo = orc.f32_bits(v) >> 16  # truncation toward zero, then the next bf16 away from zero
    vals = orc.bf16_to_f64(got)
    assert np.all((vals == orc.bf16_to_f64(lo.astype(np.uint16))) | (vals == orc.bf16_to_f64((lo + 1).astype(np.uint16))))
    # the update moves against H: mostly the weights decrease where h > 0
    hs = orc.reconstruct(c, p)
    moved = vals - wv
    assert np.sum(moved * hs) < 0


def test_agrees_with_normalized_update_at_its_step():
    rng = np.random.default_rng(5)
    d, k, r = 48, 96, 16
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    c = (rng.standard_normal((d, r)) * 1e-2).astype(np.float32)
    p = orc.qr_projection(3, k, r)
    ref, stats = orc.apply_update(w, c, p, 1e-3, 9)
    assert stats[3] == 0
    assert np.array_equal(orc.apply_scaled(w, c, p, stats[2], 9), ref)


def test_zero_step_keeps_weights():
    w, c, p = _tiny(seed=2)
    assert np.array_equal(orc.apply_scaled(w, c, p, 0.0, 5), w)


def test_mean_over_rounding_seeds_is_the_fp32_step():
    """E[W'] = v exactly under stochastic rounding; the sample mean over 400
    seeds lies within a few standard errors of v everywhere (in aggregate)."""
    w, c, p = _tiny(seed=4, d=8, k=16, r=4)
    alpha = np.float32(1e-3)
    h32 = orc.reconstruct(c, p).astype(np.float32)
    v = (orc.bf16_to_f64(w).astype(np.float32) - (alpha * h32).astype(np.float32)).astype(np.float32)
    outs = np.stack([orc.bf16_to_f64(orc.apply_scaled(w, c, p, alpha, sd)) for sd in range(400)])
    lo = orc.bf16_to_f64(orc.f32_bits(v) >> 16)
    hi = orc.bf16_to_f64((orc.f32_bits(v) >> 16) + 1)
    gap = np.abs(hi - lo)
    z = (outs.mean(axis=0) - v) / (gap / 2 / np.sqrt(400))
    assert abs(z.mean()) < 4 / np.sqrt(z.size)
    assert np.max(np.abs(z)) < 6
