"""Bit-exact parity of the rounding decisions that write W.

The update's pre-rounding value is v = fp32(w - fp32(s * h)) and its bf16
result is SR(v, r16) with r16 from the (seed, row, column) Philox stream
[page "Randomized Gradient Compression", "How it works": bf16 weights with
stochastic rounding, no fp32 copy]. The parity tests elsewhere compare W with
the oracle's update within one ulp, because the oracle's h (fp64) and the
kernel's h (fp32 MFMA sums of a two-term bf16 C) differ in their last bits.

Here the rounding is checked alone, given identical fp32 pre-round inputs:
h is the GPU's own H from rgc_test_reconstruct (the update sweep's tile code,
same operands, same MFMA order) and s is the step the call reports (or the
caller's alpha). The oracle forms v from (W, h, s) with its own fp32
arithmetic and rounds it with its own Philox stream; the result must equal
the GPU's W in every bit, through every entry point that writes W: rgc_apply
(all ranks, ragged and strided shapes), rgc_apply_batch on the full-size
Qwen3-1.7B-shaped block (sampled rows), rgc_apply_scaled (alpha) and
rgc_apply_carried (the variant that also sums the written squares).
The h and s handed to the oracle are themselves checked against the oracle's
own reconstruct and step, so the test isolates the rounding without trusting
them.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits
from_bits = synth.from_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _inputs(d, k, r, seed):
    w = synth.normal_bf16((d, k), 0.02, seed=seed)
    c = synth.normal_f32((d, r), 1e-2, seed=seed + 1)
    p = orc.qr_projection(seed, k, r) if r <= 128 else orc.rademacher_projection(seed, k, r)
    return w, c, from_bits(p)


def _expected(w_bits, h32, s, seed, row0=0):
    """The oracle's rounding of the GPU's h: SR(fp32(w - fp32(s h)), Philox bits of (seed, row, col))."""
    rows, cols = np.shape(w_bits)
    v = orc.pre_round_values(w_bits, h32, np.float32(s))
    return orc.stochastic_round(v, orc.rounding_bits(seed, rows, cols, row0=row0))


def _check_h(h32, c, p_bits):
    err = rel_frobenius(h32, orc.reconstruct(c, p_bits))
    assert err < 2e-5, err


CASES = [(256, 512, 16), (1000, 520, 48), (2048, 2048, 64), (264, 1024, 128), (128, 2048, 256),
         (64, 512, 192), (6144, 2048, 64), (2048, 6144, 64), (1000, 520, 256), (264, 1048, 192),
         (1096, 2056, 128), (40, 24, 16)]


@pytest.mark.parametrize("d,k,r", CASES)
def test_apply_rounding_bitexact(dev, d, k, r):
    w, c, p = _inputs(d, k, r, 101)
    seed, tau = 0x1234 + d * 7 + k, 1e-3
    cg, pg = c.to(dev), p.to(dev)
    h = rgc.rgc_test_reconstruct(cg, pg)
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, cg, pg, tau, seed, stats=stats)
    torch.cuda.synchronize()
    h32 = h.cpu().numpy()
    _check_h(h32, c.numpy(), bits(p))
    st = stats.cpu().numpy()
    _, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seed)
    np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
    assert st[3] == 0
    got = bits(wg)
    exp = _expected(bits(w), h32, st[2], seed)
    assert np.count_nonzero(got != exp) == 0, f"{np.count_nonzero(got != exp)} rounding mismatches"


@pytest.mark.parametrize("d,k,r,pad", [(1032, 24, 16, 8), (264, 12808, 64, 8), (200, 1040, 256, 16)])
def test_apply_rounding_bitexact_row_stride(dev, d, k, r, pad):
    w, c, p = _inputs(d, k, r, 131)
    full = synth.normal_bf16((d, k + pad), 0.02, seed=132)
    off = 8 if pad >= 16 else 0
    full[:, off:off + k] = w
    fg = full.clone().to(dev)
    wg = fg[:, off:off + k]
    seed = 0x77 + k
    cg, pg = c.to(dev), p.to(dev)
    h = rgc.rgc_test_reconstruct(cg, pg)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, cg, pg, 1e-3, seed, stats=stats)
    torch.cuda.synchronize()
    got = bits(wg.contiguous())
    exp = _expected(bits(w), h.cpu().numpy(), stats.cpu().numpy()[2], seed)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("d,k,r,alpha", [(256, 512, 16, 3e-5), (2048, 2048, 64, 1e-4), (264, 1048, 192, 2e-4),
                                         (1096, 2056, 128, 5e-6), (128, 2048, 256, 1e-3)])
def test_apply_scaled_rounding_bitexact(dev, d, k, r, alpha):
    w, c, p = _inputs(d, k, r, 141)
    seed = 0x99 + d
    cg, pg = c.to(dev), p.to(dev)
    h = rgc.rgc_test_reconstruct(cg, pg)
    wg = w.clone().to(dev)
    rgc.rgc_apply_scaled(wg, cg, pg, alpha, seed)
    torch.cuda.synchronize()
    exp = _expected(bits(w), h.cpu().numpy(), np.float32(alpha), seed)
    assert np.array_equal(bits(wg), exp)


@pytest.mark.parametrize("d,k,r", [(2048, 2048, 64), (264, 1024, 128), (1000, 520, 256)])
def test_apply_carried_rounding_bitexact(dev, d, k, r):
    """Three carried updates in a row (the first streams ||W||): every one
    rounds exactly as the oracle rounds the GPU's h with the reported s."""
    w, c, p = _inputs(d, k, r, 151)
    cg, pg = c.to(dev), p.to(dev)
    h32 = rgc.rgc_test_reconstruct(cg, pg).cpu().numpy()
    wg = w.clone().to(dev)
    wn2 = torch.zeros(1, dtype=torch.float64, device=dev)
    prev = bits(w)
    for u in range(3):
        seed = 0x500 + u
        stats = torch.zeros(4, device=dev)
        rgc.rgc_apply_carried(wg, cg, pg, 1e-3, seed, wn2, fresh=(u == 0), stats=stats)
        torch.cuda.synchronize()
        got = bits(wg)
        exp = _expected(prev, h32, stats.cpu().numpy()[2], seed)
        assert np.array_equal(got, exp), u
        # the carried norm is the squared norm of the weights written
        assert wn2.item() == pytest.approx(orc.weight_sumsq(got), rel=1e-6)
        prev = got


BLOCK_1P7B = [(2048, 2048), (1024, 2048), (1024, 2048), (2048, 2048), (6144, 2048), (6144, 2048), (2048, 6144)]


def test_apply_batch_rounding_bitexact_full_block(dev):
    """The full-size Qwen3-1.7B-shaped block through rgc_apply_batch (r = 64,
    QR projections): 48 sampled rows per matrix, the first and last included,
    every element of each compared bit for bit."""
    r, tau = 64, 1e-3
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    Ws = [(torch.randn(d, k, generator=g, device=dev) * 0.02).to(torch.bfloat16) for d, k in BLOCK_1P7B]
    Cs = [torch.randn(d, r, generator=g, device=dev) * 1e-2 for d, _ in BLOCK_1P7B]
    Ps = [torch.empty(k, r, dtype=torch.bfloat16, device=dev) for _, k in BLOCK_1P7B]
    rgc.rgc_sample_projections("qr", [(9 << 32) | m for m in range(len(Ps))], Ps)
    Hs = [rgc.rgc_test_reconstruct(c, p) for c, p in zip(Cs, Ps)]
    W0 = [bits(w) for w in Ws]
    seeds = [(3 << 40) | m for m in range(len(Ws))]
    stats = [torch.zeros(4, device=dev) for _ in Ws]
    rgc.rgc_apply_batch(Ws, Cs, Ps, tau, seeds, stats=stats)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for m, (d, k) in enumerate(BLOCK_1P7B):
        rows = np.unique(np.concatenate([[0, d - 1], rng.choice(d, 46, replace=False)]))
        s = stats[m].cpu().numpy()[2]
        h = Hs[m].cpu().numpy()
        c = Cs[m].cpu().numpy()
        p_bits = bits(Ps[m])
        got = bits(Ws[m])
        for i in rows:
            _check_h(h[i:i + 1], c[i:i + 1], p_bits)
            exp = _expected(W0[m][i:i + 1], h[i:i + 1], s, seeds[m], row0=int(i))
            assert np.array_equal(got[i:i + 1], exp), (m, int(i))


def test_nan_projection_skips_the_update(dev):
    """A projection that failed to factorize is all NaN; the sketch built from
    it is NaN, so the update is skipped (flag = 1) and W stays bit-identical."""
    d, k, r, T = 256, 512, 16, 256
    p = torch.full((k, r), float("nan"), dtype=torch.bfloat16, device=dev)
    x = synth.normal_bf16((T, k), 1.0, seed=7).to(dev)
    dd = synth.normal_bf16((T, d), 0.1, seed=8).to(dev)
    c = torch.zeros(d, r, device=dev)
    rgc.rgc_accumulate(dd, rgc.rgc_project(x, p), c)
    w = synth.normal_bf16((d, k), 0.02, seed=9)
    wg = w.clone().to(dev)
    stats = torch.zeros(4, device=dev)
    rgc.rgc_apply(wg, c, p, 1e-3, 1, stats=stats)
    torch.cuda.synchronize()
    assert stats.cpu().numpy()[3] == 1
    assert np.array_equal(bits(wg), bits(w))
