"""GPU parity: every librgc entry point against the CPU oracle on the same
seeded inputs (inputs flow oracle -> GPU only, never the other way).

Bars (floating point: bf16 inputs, fp32 accumulation):
  * Philox words, Rademacher P, the rounding stream and stochastic rounding of
    given fp32 values: bit-exact.
  * QR P: bit-exact except where the oracle's pre-rounding fp64 value lies
    within 1e-12 (relative) of a rounding boundary (then either neighbour).
  * XP = bf16(X P): relative Frobenius error <= 2e-3; every element within
    1 bf16 ulp plus 2^-20 * sum_i |x_i p_i| (the GPU sums in fp32, the oracle
    in fp64; where the terms cancel to near zero the fp32 sum error exceeds
    an ulp of the result), at most 1e-3 of the elements differing.
  * C and H: relative Frobenius error <= 2e-3.
  * W after the update: every element within 1 bf16 ulp plus s * 2^-15 *
    sum_a |c_ia p_ja| (where w and s*h cancel, h's fp32 error scaled by s can
    exceed an ulp of the tiny result), at most 1e-4 of them differing;
    ||W||, ||H|| and s within 1e-5 relative. The rounding decisions themselves
    are checked bit-exactly on given fp32 values (stochastic-round test).
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()  # fails loudly if the HIP library is missing
    return torch.device("cuda", 0)


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Random streams
# ---------------------------------------------------------------------------
def test_philox_bitexact(dev):
    rng = np.random.default_rng(0)
    n = 1 << 16
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    ctr[0] = 0
    ctr[1] = 0xFFFFFFFF
    for seed in (0, 1, 0xDEADBEEFCAFEF00D, 2**63 + 17):
        got = rgc.rgc_test_philox(seed, torch.from_numpy(ctr.view(np.int32)).to(dev))
        _sync()
        got = got.cpu().numpy().view(np.uint32)
        k0, k1 = orc.seed_to_key(seed)
        ref = np.stack(orc.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], k0, k1), axis=1)
        assert np.array_equal(got, ref), seed


def _edge_values():
    vals = np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 1.1754942e-38, 3.3895314e38, -3.3895314e38,
                     3.4028235e38, np.inf, -np.inf], dtype=np.float32)
    low = orc.bits_f32(np.array([0x3F800001, 0x3F807FFF, 0x3F808000, 0x3F80FFFF, 0xBF808000, 0x00000001,
                                 0x80007FFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x7FC00001, 0xFF800001], dtype=np.uint32))
    return np.concatenate([vals, low])


@pytest.mark.parametrize("rows,cols,row0,col0,seed", [(64, 1000, 0, 0, 0), (33, 77, 37, 1021, 12345),
                                                     (8, 4096, 5000, 8, 2**40 + 1)])
def test_stochastic_round_bitexact(dev, rows, cols, row0, col0, seed):
    rng = np.random.default_rng(seed & 0xFFFF)
    v = (rng.standard_normal((rows, cols)) * np.float64(10.0) ** rng.integers(-6, 3, (rows, cols))).astype(np.float32)
    e = _edge_values()
    v.ravel()[: e.size] = e
    rnd = orc.bits_f32(rng.integers(0, 2**32, size=rows * cols, dtype=np.uint64).astype(np.uint32)).reshape(rows, cols)
    v[rows // 2:] = rnd[rows // 2:]  # arbitrary bit patterns, including NaNs and subnormals
    got = rgc.rgc_test_stochastic_round(torch.from_numpy(v).to(dev), seed, row0, col0)
    _sync()
    ref = orc.stochastic_round(v, orc.rounding_bits(seed, rows, cols, row0, col0))
    assert np.array_equal(bits(got), ref)


def test_round_nearest_bitexact(dev):
    """The kernels' nearest-even bf16 conversion (the conversion instruction)
    against the oracle's integer definition: every sign, exponent and upper
    mantissa (all 2^16 high halves) with the low halves that decide the
    rounding (zero, just above zero, just below, at and just above the tie, all
    ones), then 2^20 arbitrary bit patterns: NaNs with payloads, infinities,
    subnormals, the overflow to infinity at the top of the range."""
    high = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    grid = (high[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(77).integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = orc.bits_f32(np.concatenate([grid, rnd]))
    got = rgc.rgc_test_round_nearest(torch.from_numpy(v).to(dev))
    _sync()
    assert np.array_equal(bits(got), orc.f32_to_bf16_rne(v))


# ---------------------------------------------------------------------------
# Projection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k,r,seed", [(512, 16, 0), (2048, 64, 5), (6144, 256, 7), (1000, 48, 9),
                                      (4096, 128, 2**40 + 3), (2048, 192, 11), (2056, 32, 1)])
def test_rademacher_bitexact(dev, k, r, seed):
    got = rgc.rgc_sample_projection("rademacher", seed, k, r, device=dev)
    _sync()
    assert np.array_equal(bits(got), orc.rademacher_projection(seed, k, r))


_qr_margin_ok = qr_margin_mismatches


@pytest.mark.parametrize("k,r,seed", [(512, 16, 0), (2048, 64, 12345), (6144, 64, 77), (4096, 128, 3),
                                      (1000, 48, 5), (2048, 32, 2**63 + 9), (12288, 128, 21)])
def test_qr_projection_bitexact(dev, k, r, seed):
    got = rgc.rgc_sample_projection("qr", seed, k, r, device=dev)
    _sync()
    nbad = _qr_margin_ok(bits(got), seed, k, r)
    assert nbad <= 2


@pytest.mark.parametrize("k,r,seed", [(64, 64, 1), (128, 64, 2), (128, 128, 3), (96, 48, 4), (32, 16, 5)])
def test_qr_projection_near_square(dev, k, r, seed):
    """k close to r: the Gaussian is far less well conditioned, so the first
    CholeskyQR pass is not orthonormal to 1e-14 and the second pass's multiply
    runs. Both sides are backward stable, so their Q differ by about
    cond(A) * 1e-16; the margin is widened to 1e-10 accordingly."""
    got = rgc.rgc_sample_projection("qr", seed, k, r, device=dev)
    _sync()
    a = orc.gaussian_matrix(seed, k, r)
    assert np.linalg.cond(a) < 1e5
    nbad = _qr_margin_ok(bits(got), seed, k, r, rel=1e-10)
    assert nbad <= 2
    pv = orc.bf16_to_f64(bits(got))
    np.testing.assert_allclose(pv.T @ pv, (k / r) * np.eye(r), atol=2e-2 * k / r)


def test_batched_projections_equal_single_draws(dev):
    shapes = [(2048, 1), (1024, 2), (6144, 3), (2048, 2**40 + 4), (4096, 5)]
    for kind in ("qr", "rademacher"):
        ps = [torch.empty((k, 64), dtype=torch.bfloat16, device=dev) for k, _ in shapes]
        rgc.rgc_sample_projections(kind, [s for _, s in shapes], ps)
        singles = [rgc.rgc_sample_projection(kind, s, k, 64, device=dev).clone() for k, s in shapes]
        _sync()
        for a, b in zip(ps, singles):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _sync()


def test_projection_repeatable(dev):
    a = rgc.rgc_sample_projection("qr", 99, 2048, 64, device=dev).clone()
    b = rgc.rgc_sample_projection("qr", 99, 2048, 64, device=dev).clone()
    c = rgc.rgc_sample_projection("qr", 100, 2048, 64, device=dev).clone()
    _sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))


# ---------------------------------------------------------------------------
# Sketch contractions
# ---------------------------------------------------------------------------
# includes k < 32 (a single, short K window), k = 2056 (a short last k chunk)
# and T < 64 (one partial token tile); one matrix per launch takes the narrow
# 128-token tiles at r = 64, 96 and 128 where its K-steps are few (e.g.
# 4096 x 2048 at r = 64), the wide 256-token tiles otherwise
PROJECT_CASES = [(256, 512, 16), (1000, 520, 48), (37, 2048, 64), (4096, 2048, 64), (300, 1024, 128),
                 (129, 512, 192), (200, 2048, 256), (64, 512, 32), (4096, 6144, 64), (20, 24, 16),
                 (100, 2056, 64), (7, 16, 16), (4096, 4096, 96)]


@pytest.mark.parametrize("T,k,r", PROJECT_CASES)
def test_project_parity(dev, T, k, r):
    x = synth.normal_bf16((T, k + 8), 1.0, seed=T * 7 + k)[:, 4:k + 4]  # row stride k + 8
    p = synth.normal_bf16((k, r), 1.0, seed=r)
    got = rgc.rgc_project(x.to(dev), p.to(dev))
    _sync()
    ref = orc.project(bits(x), bits(p))
    abs_terms = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(p)))
    assert_sum_close(bits(got), ref, abs_terms, what=f"XP {T}x{k}x{r}")
    assert rel_frobenius(orc.bf16_to_f64(bits(got)), orc.bf16_to_f64(ref)) < 2e-3


# includes T < 32 (a single, short K window) and T = 4100 (a last token
# split of 4 tokens)
ACC_CASES = [(256, 256, 16), (1000, 1000, 48), (4096, 2048, 64), (77, 520, 128), (300, 264, 192),
             (513, 1024, 256), (33, 64, 32), (4096, 6144, 64), (4096, 1024, 256), (20, 72, 16), (5, 8, 64),
             (4100, 256, 64), (4096, 4096, 96)]


@pytest.mark.parametrize("T,d,r", ACC_CASES)
def test_accumulate_parity(dev, T, d, r):
    dd = synth.normal_bf16((T, d + 16), 1e-3, seed=T + d)[:, 8:d + 8]  # row stride d + 16
    xp = synth.normal_bf16((T, r), 3.0, seed=r + 1)
    c0 = synth.normal_f32((d, r), 1e-3, seed=5)
    c = c0.clone().to(dev)
    rgc.rgc_accumulate(dd.to(dev), xp.to(dev), c)
    _sync()
    ref = orc.accumulate(c0.numpy(), bits(dd), bits(xp))
    err = rel_frobenius(c.cpu().numpy(), ref)
    assert err < 2e-3, err
    assert err < 1e-5, err  # fp32 accumulation: expect ~1e-6


def test_project_batch_parity(dev):
    """The projections of one block in one launch: q/k/v share an X, down has k = 6144."""
    T, r = 1000, 64
    xa = synth.normal_bf16((T, 2048), 1.0, seed=31)
    xd = synth.normal_bf16((T, 6144 + 8), 1.0, seed=32)[:, :6144]
    ks = [2048, 2048, 2048, 6144]
    xs = [xa, xa, xa, xd]
    ps = [synth.normal_bf16((k, r), 1.0, seed=40 + i) for i, k in enumerate(ks)]
    outs = rgc.rgc_project_batch([x.to(dev) for x in xs], [p.to(dev) for p in ps])
    _sync()
    for x, p, o in zip(xs, ps, outs):
        ref = orc.project(bits(x), bits(p))
        abs_terms = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(p)))
        assert_sum_close(bits(o), ref, abs_terms, what="XP batch")


def test_accumulate_batch_parity(dev):
    T, r = 777, 128
    ds = [2048, 1024, 1024, 6144, 264]
    dds = [synth.normal_bf16((T, d), 1e-3, seed=50 + i) for i, d in enumerate(ds)]
    xps = [synth.normal_bf16((T, r), 3.0, seed=60 + i) for i in range(len(ds))]
    c0s = [synth.normal_f32((d, r), 1e-3, seed=70 + i) for i, d in enumerate(ds)]
    cs = [c.clone().to(dev) for c in c0s]
    rgc.rgc_accumulate_batch([d.to(dev) for d in dds], [x.to(dev) for x in xps], cs)
    _sync()
    for dd, xp, c0, c in zip(dds, xps, c0s, cs):
        ref = orc.accumulate(c0.numpy(), bits(dd), bits(xp))
        assert rel_frobenius(c.cpu().numpy(), ref) < 1e-5


def test_accumulate_batch_ranges_aligned_to_tiles(dev):
    """The Qwen3-1.7B-shaped block's seven d (80 tiles of 256 columns) at a
    ragged token count: 63 K-steps per tile, the last one 16 tokens, so that
    the schedule cuts every tile into exactly three ranges (240 workgroups on
    a 256-CU part) and each tile's last range ends in the partial step."""
    T, r = 2000, 64
    ds = [2048, 1024, 1024, 2048, 6144, 6144, 2048]
    dds = [synth.normal_bf16((T, d), 1e-3, seed=150 + i) for i, d in enumerate(ds)]
    xps = [synth.normal_bf16((T, r), 3.0, seed=160 + i) for i in range(len(ds))]
    c0s = [synth.normal_f32((d, r), 1e-3, seed=170 + i) for i, d in enumerate(ds)]
    cs = [c.clone().to(dev) for c in c0s]
    rgc.rgc_accumulate_batch([d.to(dev) for d in dds], [x.to(dev) for x in xps], cs)
    _sync()
    for dd, xp, c0, c in zip(dds, xps, c0s, cs):
        ref = orc.accumulate(c0.numpy(), bits(dd), bits(xp))
        assert rel_frobenius(c.cpu().numpy(), ref) < 1e-5


@pytest.mark.parametrize("wgs", [1, 3])
def test_sketch_batches_with_whole_tiles_per_workgroup(dev, wgs):
    """Few workgroups (forced through the test hooks): each range holds whole
    tiles, ends in later items, and the first segment's sums are stored after
    the last one (ragged d and T)."""
    T, r = 300, 64
    ds = [512, 8, 264]
    dds = [synth.normal_bf16((T, d), 1e-3, seed=80 + i) for i, d in enumerate(ds)]
    xps = [synth.normal_bf16((T, r), 3.0, seed=90 + i) for i in range(len(ds))]
    c0s = [synth.normal_f32((d, r), 1e-3, seed=95 + i) for i, d in enumerate(ds)]
    cs = [c.clone().to(dev) for c in c0s]
    rgc.rgc_test_accumulate_batch_wgs(wgs, [d.to(dev) for d in dds], [x.to(dev) for x in xps], cs)
    ks = [512, 72, 264]  # r <= k; 72 ends in a partial 32-wide step
    xs = [synth.normal_bf16((T, k), 1.0, seed=100 + i) for i, k in enumerate(ks)]
    ps = [synth.normal_bf16((k, r), 1.0, seed=110 + i) for i, k in enumerate(ks)]
    outs = rgc.rgc_test_project_batch_wgs(wgs, [x.to(dev) for x in xs], [p.to(dev) for p in ps])
    _sync()
    for dd, xp, c0, c in zip(dds, xps, c0s, cs):
        assert rel_frobenius(c.cpu().numpy(), orc.accumulate(c0.numpy(), bits(dd), bits(xp))) < 1e-5
    for x, p, o in zip(xs, ps, outs):
        abs_terms = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(p)))
        assert_sum_close(bits(o), orc.project(bits(x), bits(p)), abs_terms, what=f"XP wgs={wgs}")


def test_accumulate_empty_microbatch_is_noop(dev):
    c = torch.ones(64, 16, device=dev)
    rgc.rgc_accumulate(torch.zeros(0, 64, dtype=torch.bfloat16, device=dev),
                       torch.zeros(0, 16, dtype=torch.bfloat16, device=dev), c)
    _sync()
    assert torch.equal(c, torch.ones(64, 16, device=dev))


def test_sketch_is_deterministic(dev):
    T, k, d, r = 4096, 2048, 2048, 64
    x = synth.normal_bf16((T, k), 1.0, seed=1).to(dev)
    dd = synth.normal_bf16((T, d), 1e-3, seed=2).to(dev)
    p = rgc.rgc_sample_projection("qr", 3, k, r, device=dev)
    outs = []
    for _ in range(2):
        xp = rgc.rgc_project(x, p)
        c = torch.zeros(d, r, device=dev)
        rgc.rgc_accumulate(dd, xp, c)
        rgc.rgc_accumulate(dd, xp, c)
        _sync()
        outs.append((xp.view(torch.int16).clone(), c.view(torch.int32).clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------------------
# Update
# ---------------------------------------------------------------------------
APPLY_CASES = [(256, 512, 16), (1000, 520, 48), (2048, 2048, 64), (264, 1024, 128), (128, 2048, 256),
               (64, 512, 192), (6144, 2048, 64), (2048, 6144, 64), (1024, 2048, 256),
               # ragged row blocks and column tiles at r > 128 (128-row tiles) and r = 128 (64-row tiles)
               (1000, 520, 256), (264, 1048, 192), (1096, 2056, 128)]


def _apply_inputs(d, k, r, seed):
    w = synth.normal_bf16((d, k), 0.02, seed=seed)
    c = synth.normal_f32((d, r), 1e-2, seed=seed + 1)
    p = orc.qr_projection(seed, k, r) if r <= 128 else orc.rademacher_projection(seed, k, r)
    return w, c, from_bits(p)


@pytest.mark.parametrize("d,k,r", APPLY_CASES)
def test_reconstruct_parity(dev, d, k, r):
    _, c, p = _apply_inputs(d, k, r, 3)
    h = rgc.rgc_test_reconstruct(c.to(dev), p.to(dev))
    _sync()
    ref = orc.reconstruct(c.numpy(), bits(p))
    err = rel_frobenius(h.cpu().numpy(), ref)
    assert err < 2e-3, err
    assert err < 2e-5, err  # C split in two bf16 terms: expect a few 1e-6


@pytest.mark.parametrize("d,k,r", APPLY_CASES)
def test_apply_parity(dev, d, k, r):
    w, c, p = _apply_inputs(d, k, r, 11)
    seed, tau = 0xABCDEF + d, 1e-3
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, c.to(dev), p.to(dev), tau, seed, stats=stats)
    _sync()
    ref_w, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seed)
    st = stats.cpu().numpy()
    assert st[3] == 0 and ref_stats[3] == 0
    np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
    abs_terms = np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T
    assert_update_close(bits(wg), ref_w, ref_stats[2], abs_terms, what=f"W {d}x{k}x{r}")
    # the update actually moved the weights
    assert np.count_nonzero(bits(wg) != bits(w)) > 0.1 * d * k


@pytest.mark.parametrize("d,k,r,pad", [(1032, 24, 16, 8), (2056, 4104, 48, 24), (264, 12808, 64, 8),
                                       (776, 136, 32, 16), (136, 1048, 128, 8), (200, 1040, 256, 16)])
def test_apply_parity_row_stride_and_chunking(dev, d, k, r, pad):
    """W as a view with row stride k + pad; shapes whose norms split into
    several C-row and P-row chunks with ragged ends, and W chunks that start
    mid-row (k = 24, 136: fewer than 256 chunks of 8 per row)."""
    w, c, p = _apply_inputs(d, k, r, 21)
    full = synth.normal_bf16((d, k + pad), 0.02, seed=22)
    off = 8 if pad >= 16 else 0  # keeps W 16-byte aligned
    full[:, off:off + k] = w
    fg = full.clone().to(dev)
    wg = fg[:, off:off + k]
    seed, tau = 0x5151 + k, 1e-3
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, c.to(dev), p.to(dev), tau, seed, stats=stats)
    _sync()
    ref_w, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seed)
    st = stats.cpu().numpy()
    assert st[3] == 0 and ref_stats[3] == 0
    np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
    abs_terms = np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T
    assert_update_close(bits(wg.contiguous()), ref_w, ref_stats[2], abs_terms, what=f"W {d}x{k}x{r}+{pad}")
    # the padding columns are untouched
    got_full = bits(fg)
    ref_full = bits(full)
    assert np.array_equal(got_full[:, :off], ref_full[:, :off])
    assert np.array_equal(got_full[:, off + k:], ref_full[:, off + k:])


def test_apply_zero_sketch_leaves_weights(dev):
    d, k, r = 256, 512, 16
    w, _, p = _apply_inputs(d, k, r, 4)
    wg = w.clone().to(dev)
    stats = torch.full((4,), -1.0, device=dev)
    rgc.rgc_apply(wg, torch.zeros(d, r, device=dev), p.to(dev), 1e-3, 1, stats=stats)
    _sync()
    assert np.array_equal(bits(wg), bits(w))
    st = stats.cpu().numpy()
    assert st[1] == 0 and st[2] == 0 and st[3] == 1


def test_apply_nonfinite_sketch_leaves_weights(dev):
    d, k, r = 256, 512, 16
    w, c, p = _apply_inputs(d, k, r, 5)
    c[3, 2] = float("inf")
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, c.to(dev), p.to(dev), 1e-3, 1, stats=stats)
    _sync()
    assert np.array_equal(bits(wg), bits(w))
    assert stats.cpu().numpy()[3] == 1


def test_apply_is_deterministic_and_seeded(dev):
    d, k, r = 2048, 2048, 64
    w, c, p = _apply_inputs(d, k, r, 6)
    outs = []
    for seed in (7, 7, 8):
        wg = w.clone().to(dev)
        rgc.rgc_apply(wg, c.to(dev), p.to(dev), 1e-3, seed)
        _sync()
        outs.append(bits(wg))
    assert np.array_equal(outs[0], outs[1])
    assert not np.array_equal(outs[0], outs[2])


def test_apply_batch_matches_single_applies(dev):
    """One batched call over a block's shapes gives every matrix exactly the
    bits (and stats) of its own rgc_apply, and matches the oracle."""
    r, tau = 64, 1e-3
    shapes = [(2048, 2048), (1024, 2048), (6144, 2048), (2048, 6144), (264, 520)]
    items = [_apply_inputs(d, k, r, 40 + i) for i, (d, k) in enumerate(shapes)]
    seeds = [(5 << 32) | i for i in range(len(shapes))]
    wb = [w.clone().to(dev) for w, _, _ in items]
    cs = [c.to(dev) for _, c, _ in items]
    ps = [p.to(dev) for _, _, p in items]
    stats_b = [torch.zeros(4, device=dev) for _ in shapes]
    rgc.rgc_apply_batch(wb, cs, ps, tau, seeds, stats=stats_b)
    for i, (w, c, p) in enumerate(items):
        ws_ = w.clone().to(dev)
        st = torch.zeros(4, device=dev)
        rgc.rgc_apply(ws_, cs[i], ps[i], tau, seeds[i], stats=st)
        _sync()
        assert np.array_equal(bits(ws_), bits(wb[i])), shapes[i]
        assert torch.equal(st, stats_b[i])
    d, k = shapes[-1]
    w, c, p = items[-1]
    ref_w, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seeds[-1])
    np.testing.assert_allclose(stats_b[-1].cpu().numpy()[:3], ref_stats[:3], rtol=1e-5)
    abs_terms = np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T
    assert_update_close(bits(wb[-1]), ref_w, ref_stats[2], abs_terms, what="W batch")


def test_apply_batch_skips_only_flagged_matrix(dev):
    r = 16
    items = [_apply_inputs(256, 512, r, 50), _apply_inputs(256, 512, r, 51)]
    wb = [w.clone().to(dev) for w, _, _ in items]
    cs = [torch.zeros(256, r, device=dev), items[1][1].to(dev)]  # first sketch is zero
    ps = [p.to(dev) for _, _, p in items]
    stats = [torch.zeros(4, device=dev), torch.zeros(4, device=dev)]
    rgc.rgc_apply_batch(wb, cs, ps, 1e-3, [1, 2], stats=stats)
    _sync()
    assert np.array_equal(bits(wb[0]), bits(items[0][0]))
    assert stats[0].cpu().numpy()[3] == 1 and stats[1].cpu().numpy()[3] == 0
    assert not np.array_equal(bits(wb[1]), bits(items[1][0]))


# ---------------------------------------------------------------------------
# End to end: the small single-layer case (d=256, k=512, r=16, 4 x 256 tokens)
# ---------------------------------------------------------------------------
def test_end_to_end_small_layer(dev):
    d, k, r, mb, n_mb, tau, seed = 256, 512, 16, 256, 4, 1e-3, 0
    x = synth.normal_bf16((mb * n_mb, k), 1.0, seed=1000)
    dd = synth.normal_bf16((mb * n_mb, d), 0.1, seed=1001)  # variance 1e-2
    w = synth.normal_bf16((d, k), 0.02, seed=1002)
    ref_p, ref_c, ref_w, ref_stats = orc.sketch_update(
        "qr", r, seed, seed, bits(w), [bits(x[i * mb:(i + 1) * mb]) for i in range(n_mb)],
        [bits(dd[i * mb:(i + 1) * mb]) for i in range(n_mb)], tau)
    p = rgc.rgc_sample_projection("qr", seed, k, r, device=dev)
    c = torch.zeros(d, r, device=dev)
    xg, dg = x.to(dev), dd.to(dev)
    for i in range(n_mb):
        xp = rgc.rgc_project(xg[i * mb:(i + 1) * mb], p)
        rgc.rgc_accumulate(dg[i * mb:(i + 1) * mb], xp, c)
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, c, p, tau, seed, stats=stats)
    _sync()
    assert _qr_margin_ok(bits(p), seed, k, r) == 0
    assert rel_frobenius(c.cpu().numpy(), ref_c) < 2e-3
    np.testing.assert_allclose(stats.cpu().numpy()[:3], ref_stats[:3], rtol=1e-4)
    abs_terms = np.abs(ref_c.astype(np.float64)) @ np.abs(orc.bf16_to_f64(ref_p)).T
    assert_update_close(bits(wg), ref_w, ref_stats[2], abs_terms, rel_h=2.0**-12, max_mismatch_frac=1e-3,
                        what="W end to end")
