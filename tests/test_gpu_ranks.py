"""GPU parity at every supported rank: 4 and 8, and every multiple of 16 up
to 256 (any rank r << min(d, k) [page "LoGRA: Low-Rank Gradient Sketches",
"The Core Move"]; its rank sweep starts at 4 [page "LoGRA: Scaling LLM
Reinforcement Learning with Low-Rank Gradient Sketches", "Main Findings"]).
Ranks 4 and 8 run the small-rank kernels (VALU sums, fp64 Gram norms);
ranks whose count of 16-column blocks is odd above 128 (144, 176, 208, 240)
run the sketch contractions at a padded compute width; 80, 96, 112 take the
one-wave split and the 64-row update tiles. Shapes are ragged (T, d, k not
multiples of the tiles) so that every path through the edges runs.

Bars as in test_gpu_parity.py: XP within 1 ulp + 2^-20 sum|xp| (<= 1e-3 of
elements differing), C and H within 1e-5 / 2e-5 relative Frobenius, W within
the update bar and its rounding bit-exact given the GPU's own h and s,
Rademacher P bit-exact, QR P under the margin rule.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_sum_close, assert_update_close, qr_margin_mismatches, rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits
from_bits = synth.from_numpy_bits
RANKS = [4, 8] + list(range(16, 257, 16))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


@pytest.mark.parametrize("r", RANKS)
def test_project_every_rank(dev, r):
    T, k = 333, max(520, r + 8)
    x = synth.normal_bf16((T, k), 1.0, seed=r + 1)
    p = synth.normal_bf16((k, r), 1.0, seed=r + 2)
    got = rgc.rgc_project(x.to(dev), p.to(dev))
    torch.cuda.synchronize()
    ref = orc.project(bits(x), bits(p))
    abs_terms = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(p)))
    assert_sum_close(bits(got), ref, abs_terms, what=f"XP r={r}")


@pytest.mark.parametrize("r", RANKS)
def test_accumulate_every_rank(dev, r):
    T, d = 333, 264
    dd = synth.normal_bf16((T, d), 1e-3, seed=r + 3)
    xp = synth.normal_bf16((T, r), 3.0, seed=r + 4)
    c0 = synth.normal_f32((d, r), 1e-3, seed=r + 5)
    c = c0.clone().to(dev)
    rgc.rgc_accumulate(dd.to(dev), xp.to(dev), c)
    torch.cuda.synchronize()
    assert rel_frobenius(c.cpu().numpy(), orc.accumulate(c0.numpy(), bits(dd), bits(xp))) < 1e-5


@pytest.mark.parametrize("r", RANKS)
def test_batched_sketch_every_rank(dev, r):
    """A two-item batch per contraction (ragged widths), so that ranges cross
    items at the padded widths too."""
    T = 200
    ks = [max(264, r), max(1048, r)]
    xs = [synth.normal_bf16((T, k), 1.0, seed=r + 10 + i) for i, k in enumerate(ks)]
    ps = [synth.normal_bf16((k, r), 1.0, seed=r + 20 + i) for i, k in enumerate(ks)]
    outs = rgc.rgc_project_batch([x.to(dev) for x in xs], [p.to(dev) for p in ps])
    ds = [520, 72]
    dds = [synth.normal_bf16((T, d), 1e-3, seed=r + 30 + i) for i, d in enumerate(ds)]
    xps = [synth.normal_bf16((T, r), 3.0, seed=r + 40 + i) for i in range(2)]
    c0s = [synth.normal_f32((d, r), 1e-3, seed=r + 50 + i) for i, d in enumerate(ds)]
    cs = [c.clone().to(dev) for c in c0s]
    rgc.rgc_accumulate_batch([d.to(dev) for d in dds], [x.to(dev) for x in xps], cs)
    torch.cuda.synchronize()
    for x, p, o in zip(xs, ps, outs):
        abs_terms = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(p)))
        assert_sum_close(bits(o), orc.project(bits(x), bits(p)), abs_terms, what=f"XP batch r={r}")
    for dd, xp, c0, c in zip(dds, xps, c0s, cs):
        assert rel_frobenius(c.cpu().numpy(), orc.accumulate(c0.numpy(), bits(dd), bits(xp))) < 1e-5


def _apply_inputs(d, k, r, seed):
    w = synth.normal_bf16((d, k), 0.02, seed=seed)
    c = synth.normal_f32((d, r), 1e-2, seed=seed + 1)
    p = orc.qr_projection(seed, k, r) if r <= 128 else orc.rademacher_projection(seed, k, r)
    return w, c, from_bits(p)


@pytest.mark.parametrize("r", RANKS)
def test_apply_every_rank(dev, r):
    d, k = 264, 1048
    w, c, p = _apply_inputs(d, k, r, 7 * r)
    seed, tau = 0xAB00 + r, 1e-3
    cg, pg = c.to(dev), p.to(dev)
    h = rgc.rgc_test_reconstruct(cg, pg)
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, cg, pg, tau, seed, stats=stats)
    torch.cuda.synchronize()
    h32 = h.cpu().numpy()
    assert rel_frobenius(h32, orc.reconstruct(c.numpy(), bits(p))) < 2e-5
    ref_w, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seed)
    st = stats.cpu().numpy()
    np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
    abs_terms = np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T
    assert_update_close(bits(wg), ref_w, ref_stats[2], abs_terms, what=f"W r={r}")
    v = orc.pre_round_values(bits(w), h32, np.float32(st[2]))
    assert np.array_equal(bits(wg), orc.stochastic_round(v, orc.rounding_bits(seed, d, k)))


@pytest.mark.parametrize("r", RANKS)
def test_apply_scaled_every_rank(dev, r):
    d, k = 136, 520
    w, c, p = _apply_inputs(d, k, r, 11 * r)
    cg, pg = c.to(dev), p.to(dev)
    h = rgc.rgc_test_reconstruct(cg, pg)
    wg = w.clone().to(dev)
    rgc.rgc_apply_scaled(wg, cg, pg, 1e-4, 5 + r)
    torch.cuda.synchronize()
    v = orc.pre_round_values(bits(w), h.cpu().numpy(), np.float32(1e-4))
    assert np.array_equal(bits(wg), orc.stochastic_round(v, orc.rounding_bits(5 + r, d, k)))


@pytest.mark.parametrize("r", RANKS)
def test_rademacher_every_rank(dev, r):
    k = 1000
    got = rgc.rgc_sample_projection("rademacher", 100 + r, k, r, device=dev)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), orc.rademacher_projection(100 + r, k, r))


@pytest.mark.parametrize("r", [r for r in RANKS if r <= 128])
def test_qr_every_rank(dev, r):
    k = 2056
    got = rgc.rgc_sample_projection("qr", 200 + r, k, r, device=dev)
    torch.cuda.synchronize()
    assert qr_margin_mismatches(bits(got), 200 + r, k, r) <= 2


@pytest.mark.parametrize("r", [4, 8, 16, 112, 144])
def test_apply_carried_every_path(dev, r):
    """Three carried updates (the first streams ||W||) through the small-rank,
    Gram-form and rebuilt-norm paths: each rounds exactly the GPU's own h with
    the reported s, and the carried value is the written weights' ||W||^2."""
    d, k = 264, 1048
    w, c, p = _apply_inputs(d, k, r, 13 * r)
    cg, pg = c.to(dev), p.to(dev)
    h32 = rgc.rgc_test_reconstruct(cg, pg).cpu().numpy()
    wg = w.clone().to(dev)
    wn2 = torch.zeros(1, dtype=torch.float64, device=dev)
    prev = bits(w)
    for u in range(3):
        stats = torch.zeros(4, device=dev)
        rgc.rgc_apply_carried(wg, cg, pg, 1e-3, 77 + u, wn2, fresh=(u == 0), stats=stats)
        torch.cuda.synchronize()
        st = stats.cpu().numpy()
        _, ref_stats = orc.apply_update(prev, c.numpy(), bits(p), 1e-3, 77 + u)
        np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
        got = bits(wg)
        v = orc.pre_round_values(prev, h32, np.float32(st[2]))
        assert np.array_equal(got, orc.stochastic_round(v, orc.rounding_bits(77 + u, d, k))), u
        assert wn2.item() == pytest.approx(orc.weight_sumsq(got), rel=1e-6)
        prev = got


@pytest.mark.parametrize("r", [4, 8])
def test_small_rank_zero_sketch_skips(dev, r):
    d, k = 136, 520
    w, _, p = _apply_inputs(d, k, r, 3)
    wg = w.clone().to(dev)
    stats = torch.full((4,), -1.0, device=dev)
    rgc.rgc_apply(wg, torch.zeros(d, r, device=dev), p.to(dev), 1e-3, 1, stats=stats)
    torch.cuda.synchronize()
    assert np.array_equal(bits(wg), bits(w))
    st = stats.cpu().numpy()
    assert st[1] == 0 and st[2] == 0 and st[3] == 1


@pytest.mark.parametrize("r", [4, 16, 64, 256])
def test_logra_fixed_rademacher_loop(dev, r):
    """The LoGRA loop at its sweep's ranks [page "LoGRA: Low-Rank Gradient
    Sketches", "Minimal Causal Code"]: a Rademacher P from a seed, a sketch
    accumulated over microbatches, the fixed-step update W -= alpha C P^T;
    against the oracle's loop (P bit-exact, C within 1e-4, W within the
    update bar)."""
    d, k, T, mb, alpha, seed = 264, 1048, 512, 128, 2e-5, 31
    x = synth.normal_bf16((T, k), 1.0, seed=r + 60)
    dd = synth.normal_bf16((T, d), 1e-3, seed=r + 61)
    w = synth.normal_bf16((d, k), 0.02, seed=r + 62)
    p_ref = orc.rademacher_projection(seed, k, r)
    c_ref = np.zeros((d, r), np.float32)
    for i in range(0, T, mb):
        c_ref = orc.accumulate(c_ref, bits(dd[i:i + mb]), orc.project(bits(x[i:i + mb]), p_ref))
    w_ref = orc.apply_scaled(bits(w), c_ref, p_ref, np.float32(alpha), seed + 1)
    p = rgc.rgc_sample_projection("rademacher", seed, k, r, device=dev)
    c = torch.zeros(d, r, device=dev)
    xg, dg = x.to(dev), dd.to(dev)
    for i in range(0, T, mb):
        rgc.rgc_accumulate(dg[i:i + mb], rgc.rgc_project(xg[i:i + mb], p), c)
    wg = w.clone().to(dev)
    rgc.rgc_apply_scaled(wg, c, p, alpha, seed + 1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(p), p_ref)
    assert rel_frobenius(c.cpu().numpy(), c_ref) < 1e-4
    abs_terms = np.abs(c_ref.astype(np.float64)) @ np.abs(orc.bf16_to_f64(p_ref)).T
    assert_update_close(bits(wg), w_ref, alpha, abs_terms, max_mismatch_frac=1e-3, what=f"LoGRA W r={r}")
