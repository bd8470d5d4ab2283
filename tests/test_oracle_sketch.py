"""Pins for the oracle's projection, sketch and update (CPU only).

Each test checks the oracle against something other than itself: the QR
uniqueness conditions and a second QR algorithm, closed-form moments of the
estimator, brute force on tiny inputs, the Gram identity for ||C P^T||, rank
bounds, and the values the pages print for the memory model.
"""
import json
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cholesky_qr2(a):
    """A different route to the same Q: two CholeskyQR passes (Fukaya et al.)."""
    q = a
    for _ in range(2):
        rr = np.linalg.cholesky(q.T @ q).T  # upper, positive diagonal
        q = np.linalg.solve(rr.T, q.T).T
    return q


@pytest.mark.parametrize("k,r,seed", [(512, 16, 0), (2048, 64, 5), (300, 48, 9)])
def test_frame_satisfies_qr_uniqueness_conditions(k, r, seed):
    a = orc.gaussian_matrix(seed, k, r)
    q = orc.orthonormal_frame(a)
    assert np.abs(q.T @ q - np.eye(r)).max() < 1e-13
    rr = q.T @ a
    assert np.abs(np.tril(rr, -1)).max() < 1e-12 * np.abs(a).max() * np.sqrt(k)
    assert np.all(np.diag(rr) > 0)
    assert np.abs(q @ np.triu(rr) - a).max() < 1e-12 * np.abs(a).max() * np.sqrt(k)
    # the same Q by CholeskyQR2
    assert np.abs(_cholesky_qr2(a) - q).max() < 1e-13


@pytest.mark.parametrize("k,r", [(512, 16), (2048, 64), (6144, 64), (4096, 128)])
def test_qr_projection_gram_is_scaled_identity(k, r):
    pre = orc.qr_projection_preround(11, k, r)
    g = pre.T @ pre
    assert np.abs(g - (k / r) * np.eye(r)).max() < 1e-12 * (k / r)
    stored = orc.bf16_to_f64(orc.qr_projection(11, k, r))
    gs = stored.T @ stored
    assert np.abs(gs - (k / r) * np.eye(r)).max() < 1e-3 * (k / r)
    # column norms sqrt(k/r); storage rounding is fp64 -> fp32 -> bf16
    assert np.array_equal(orc.qr_projection(11, k, r), orc.f32_to_bf16_rne(pre.astype(np.float32)))


def _ideal_projections(kind, seeds, k, r):
    if kind == "qr":
        return np.sqrt(k / r) * orc.orthonormal_frame(orc.gaussian_matrix(seeds, k, r))
    signs = np.where(orc.bf16_to_f64(orc.rademacher_projection(seeds, k, r)) < 0, -1.0, 1.0)
    return signs / np.sqrt(r)


@pytest.mark.parametrize("kind,factor", [("qr", lambda k, r: k / r - 1), ("rademacher", lambda k, r: (k - 1) / r)])
def test_estimator_unbiased_with_closed_form_error(kind, factor):
    """Mean of H = G P P^T over draws tends to G [RGC, footnote 1]; the mean
    squared error per draw is the closed form (k/r - 1)||G||^2 (QR frame) or
    ((k-1)/r)||G||^2 (random signs)."""
    d, k, r, n = 4, 8, 2, 60000
    rng = np.random.default_rng(0)
    g = rng.standard_normal((d, k))
    seeds = np.arange(1, n + 1, dtype=np.uint64) * np.uint64(7919)
    p = _ideal_projections(kind, seeds, k, r)  # n x k x r
    h = g[None] @ p @ np.transpose(p, (0, 2, 1))  # n x d x k
    err = np.sum((h - g[None]) ** 2, axis=(1, 2)) / np.sum(g * g)
    se = err.std() / np.sqrt(n)
    assert abs(err.mean() - factor(k, r)) < 4 * se, (err.mean(), factor(k, r), se)
    z = (h.mean(axis=0) - g) / (h.std(axis=0) / np.sqrt(n))
    assert np.abs(z).max() < 5.0
    # E[P P^T] = I_k
    ppt = (p @ np.transpose(p, (0, 2, 1))).mean(axis=0)
    assert np.abs(ppt - np.eye(k)).max() < 0.05


def test_brute_force_sketch_equals_projected_gradient():
    """[LoGRA-M] S = G A^T is reached without forming G: C P^T == G P P^T."""
    rng = np.random.default_rng(1)
    d, k, r, t = 4, 8, 2, 16
    x = orc.f32_to_bf16_rne(rng.standard_normal((t, k)).astype(np.float32))
    dd = orc.f32_to_bf16_rne(rng.standard_normal((t, d)).astype(np.float32))
    p = orc.qr_projection(3, k, r)
    x64, d64, p64 = orc.bf16_to_f64(x), orc.bf16_to_f64(dd), orc.bf16_to_f64(p)
    g = d64.T @ x64  # the dense gradient, formed only here
    # ideal mode: no intermediate rounding
    c_ideal = d64.T @ (x64 @ p64)
    assert np.abs(c_ideal @ p64.T - g @ p64 @ p64.T).max() < 1e-12 * np.abs(g).max()
    # contract mode: the oracle's rounded steps stay within bf16-level error
    c = orc.accumulate(np.zeros((d, r), np.float32), dd, orc.project(x, p))
    rel = np.linalg.norm(c - g @ p64) / np.linalg.norm(g @ p64)
    assert rel < 2**-7
    hrel = np.linalg.norm(orc.reconstruct(c, p) - g @ p64 @ p64.T) / np.linalg.norm(g @ p64 @ p64.T)
    assert hrel < 2**-7


def test_microbatch_sum_equals_whole_batch():
    """Accumulating four microbatches equals one pass over all tokens (up to fp32)."""
    rng = np.random.default_rng(2)
    d, k, r, t = 32, 64, 16, 256
    x = orc.f32_to_bf16_rne(rng.standard_normal((t, k)).astype(np.float32))
    dd = orc.f32_to_bf16_rne((0.1 * rng.standard_normal((t, d))).astype(np.float32))
    p = orc.qr_projection(4, k, r)
    xp = orc.project(x, p)
    c4 = np.zeros((d, r), np.float32)
    for m in range(4):
        c4 = orc.accumulate(c4, dd[m * 64:(m + 1) * 64], xp[m * 64:(m + 1) * 64])
    c1 = orc.accumulate(np.zeros((d, r), np.float32), dd, xp)
    assert np.abs(c4 - c1).max() <= 4 * np.finfo(np.float32).eps * np.abs(c1).max()
    assert np.array_equal(orc.project(x[:64], p), xp[:64])


def test_norm_of_update_by_gram_identity():
    """||C P^T||_F^2 = sum_ab (C^T C)_ab (P^T P)_ab, the norm the apply reports."""
    rng = np.random.default_rng(3)
    d, k, r = 96, 200, 32
    c = (rng.standard_normal((d, r)) * 1e-3).astype(np.float32)
    p = orc.qr_projection(8, k, r)
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    _, stats = orc.apply_update(w, c, p, 1e-3, 1)
    c64, p64 = c.astype(np.float64), orc.bf16_to_f64(p)
    nh = np.sqrt(np.sum((c64.T @ c64) * (p64.T @ p64)))
    nw = np.sqrt(np.sum(orc.bf16_to_f64(w) ** 2))
    assert abs(stats[1] / nh - 1) < 1e-6
    assert abs(stats[0] / nw - 1) < 1e-6
    assert abs(stats[2] / (1e-3 * nw / nh) - 1) < 1e-6
    assert stats[3] == 0


def test_normalized_step_size_sign_and_unbiased_rounding():
    """[RGC, "How it works"]: before rounding W moves by tau*||W|| against H;
    after stochastic rounding the mean over rounding seeds is that value."""
    rng = np.random.default_rng(4)
    d, k, r, tau = 64, 128, 16, 1e-3
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    c = (rng.standard_normal((d, r)) * 1e-2).astype(np.float32)
    p = orc.qr_projection(5, k, r)
    h = orc.reconstruct(c, p)
    _, stats = orc.apply_update(w, c, p, tau, 0)
    v = orc.pre_round_values(w, h.astype(np.float32), stats[2])
    w64 = orc.bf16_to_f64(w)
    step = v.astype(np.float64) - w64
    assert abs(np.linalg.norm(step) / (tau * np.linalg.norm(w64)) - 1) < 1e-3
    assert np.sum(step * h) < 0 and abs(np.sum(step * h) / (np.linalg.norm(step) * np.linalg.norm(h)) + 1) < 1e-3
    outs = np.stack([orc.bf16_to_f64(orc.apply_update(w, c, p, tau, sd)[0]) for sd in range(200)])
    mean_err = outs.mean(axis=0) - v
    ulp = np.abs(orc.bf16_to_f64(orc.f32_bits(v) >> 16 | 0) - orc.bf16_to_f64((orc.f32_bits(v) >> 16) + 1))
    z = mean_err / (ulp / 2 / np.sqrt(200))
    assert abs(z.mean()) < 5 / np.sqrt(z.size) * 2
    # stored step tracks the exact one: sum of realised moves vs the intended
    realised = (outs - w64[None]).mean(axis=0)
    assert abs(np.sum(realised * step) / np.sum(step * step) - 1) < 0.02


def test_round_to_nearest_would_erase_most_updates():
    """The pages' rationale for stochastic rounding, at the small single-layer
    scale (W ~ N(0, 0.02^2), tau = 1e-3): nearest rounding keeps most weights
    where they were, while stochastic rounding moves them correctly on average."""
    rng = np.random.default_rng(5)
    d, k, r = 256, 512, 16
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    c = (rng.standard_normal((d, r))).astype(np.float32)
    p = orc.qr_projection(0, k, r)
    h = orc.reconstruct(c, p).astype(np.float32)
    _, stats = orc.apply_update(w, c, p, 1e-3, 0)
    v = orc.pre_round_values(w, h, stats[2])
    changed_rne = np.mean(orc.f32_to_bf16_rne(v) != w)
    assert 0.1 < changed_rne < 0.35
    w_sr, _ = orc.apply_update(w, c, p, 1e-3, 0)
    moved = orc.bf16_to_f64(w_sr) - orc.bf16_to_f64(w)
    intended = v.astype(np.float64) - orc.bf16_to_f64(w)
    assert abs(np.sum(moved * intended) / np.sum(intended * intended) - 1) < 0.05


def test_rank_of_updates():
    """[LoGRA-M]: one update has rank <= r; with a fresh projection per step the
    sum of U updates reaches rank U*r, with a fixed one it stays at r."""
    rng = np.random.default_rng(6)
    d = k = 256
    r, u = 16, 10
    total_fresh = np.zeros((d, k))
    total_fixed = np.zeros((d, k))
    p_fixed = orc.bf16_to_f64(orc.qr_projection(1000, k, r))
    for step in range(u):
        g = rng.standard_normal((d, k))
        p = orc.bf16_to_f64(orc.qr_projection(step, k, r))
        h = (g @ p) @ p.T
        assert np.linalg.matrix_rank(h) == r
        total_fresh += h
        total_fixed += (g @ p_fixed) @ p_fixed.T
    assert np.linalg.matrix_rank(total_fresh) == min(u * r, d, k)
    assert np.linalg.matrix_rank(total_fixed) == r


def test_zero_sketch_skips_the_update():
    rng = np.random.default_rng(7)
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((16, 40))).astype(np.float32))
    p = orc.qr_projection(1, 40, 16)
    w2, stats = orc.apply_update(w, np.zeros((16, 16), np.float32), p, 1e-3, 3)
    assert np.array_equal(w, w2)
    assert stats[3] == 1 and stats[2] == 0 and stats[1] == 0


def test_memory_model_matches_printed_predictions():
    """[RGC, "Memory you can predict"]: the predicted savings over LoRA follow
    from an fp32 d x r sketch and a bf16 k x r projection per matrix, against
    16 bytes per LoRA adapter parameter; the state is about a fifth of LoRA's."""
    gold = json.load(open(os.path.join(GOLDEN, "memory_model.json")))
    gib = float(2**30)
    for model, ranks in gold["predicted_saving_gib"].items():
        spec = gold["models"][model]
        for r_str, printed in ranks.items():
            r = int(r_str)
            lora = sum(16 * r * (d + k) for d, k in spec["matrices"]) * spec["layers"]
            rgc = sum(4 * d * r + 2 * k * r for d, k in spec["matrices"]) * spec["layers"]
            assert round((lora - rgc) / gib, 2) == printed, (model, r, (lora - rgc) / gib)
            assert 0.15 < rgc / lora < 0.25
    ex = gold["sketch_example"]
    assert 4 * ex["d"] * ex["r"] == ex["sketch_mib"] * 2**20
    assert 4 * ex["d"] * ex["k"] == ex["dense_mib"] * 2**20


def test_apply_handles_ragged_shapes():
    rng = np.random.default_rng(8)
    d, k, r = 13, 37, 16
    w = orc.f32_to_bf16_rne((0.02 * rng.standard_normal((d, k))).astype(np.float32))
    c = rng.standard_normal((d, r)).astype(np.float32)
    p = orc.rademacher_projection(2, k, r)
    w2, stats = orc.apply_update(w, c, p, 1e-2, 9)
    assert w2.shape == (d, k) and stats[3] == 0
    assert np.mean(w2 != w) > 0.3
