"""GPU parity of the normalized update with a carried ||W|| (rgc_apply_carried,
rgc_apply_carried_batch), through the C ABI.

The normalized step of [RGC] ("How it works") scales by ||W||_F. Here the
update sums the squares of the bf16 weights it writes and hands that value to
the next call, which then reads W only once. Checked:
  * a chain of three updates (the first streams ||W|| from W, the next two
    carry it) against the oracle's own chain: the weights with the bar of the
    normalized update, the reported norms, and the carried value against the
    oracle's ||W'||^2 of its own new weights;
  * the carried chain against the plain rgc_apply chain on the GPU: the same
    step s up to its last bit, and then the same weights;
  * a skipped update (zero sketch) keeps the weights and the carried value;
  * a batch gives each matrix the bits and the value it gets alone.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_update_close

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits
from_bits = synth.from_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _w_p(d, k, r, seed):
    w = synth.normal_bf16((d, k), 0.02, seed=seed)
    p = orc.qr_projection(seed, k, r) if r <= 128 else orc.rademacher_projection(seed, k, r)
    return w, from_bits(p)


def _abs_terms(c, p):
    return np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T


# r = 16 .. 256 (Gram-form norms up to 128, rebuilt norms above), ragged row
# blocks and column tiles
CASES = [(256, 512, 16), (1000, 520, 48), (2048, 2048, 64), (264, 1024, 128), (1096, 2056, 128),
         (1000, 520, 256), (264, 1048, 192)]


@pytest.mark.parametrize("d,k,r", CASES)
def test_carried_chain_parity(dev, d, k, r):
    print(f"carried chain {d}x{k} r={r}", flush=True)
    w, p = _w_p(d, k, r, 31)
    tau = 1e-3
    wg = w.clone().to(dev)
    wn = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
    ref = bits(w)
    for step in range(3):
        c = synth.normal_f32((d, r), 1e-2, seed=40 + step)
        seed = 0x77 + 13 * step + d
        got_prev = bits(wg)
        stats = torch.zeros(4, device=dev)
        rgc.rgc_apply_carried(wg, c.to(dev), p.to(dev), tau, seed, wn, fresh=(step == 0), stats=stats)
        torch.cuda.synchronize()
        ref_new, ref_stats = orc.apply_update(ref, c.numpy(), bits(p), tau, seed)
        st = stats.cpu().numpy()
        assert st[3] == 0 and ref_stats[3] == 0
        np.testing.assert_allclose(st[:3], ref_stats[:3], rtol=1e-5)
        assert_update_close(bits(wg), ref_new, ref_stats[2], _abs_terms(c, p), max_mismatch_frac=1e-4 * (step + 1),
                            what=f"step {step}: W {d}x{k}x{r}",
                            prev_got_bits=got_prev if step else None, prev_ref_bits=ref if step else None)
        assert np.count_nonzero(bits(wg) != got_prev) > 0.1 * d * k
        np.testing.assert_allclose(wn.item(), orc.weight_sumsq(ref_new), rtol=1e-5)
        ref = ref_new


@pytest.mark.parametrize("d,k,r", [(2048, 2048, 64), (1096, 2056, 128), (1000, 520, 256)])
def test_carried_chain_matches_plain_apply(dev, d, k, r):
    """Same inputs through rgc_apply and through the carried path: the norms
    differ only in summation order, so s agrees to its last bit (here, and
    to within one fp32 ulp in general) and with an equal s the bits are
    equal."""
    print(f"carried vs plain {d}x{k} r={r}", flush=True)
    w, p = _w_p(d, k, r, 5)
    pg = p.to(dev)
    wa, wb = w.clone().to(dev), w.clone().to(dev)
    wn = torch.zeros(1, dtype=torch.float64, device=dev)
    fresh = True
    for step in range(3):
        c = synth.normal_f32((d, r), 1e-2, seed=90 + step).to(dev)
        seed = 0x99 + step
        sa, sb = torch.zeros(4, device=dev), torch.zeros(4, device=dev)
        rgc.rgc_apply(wa, c, pg, 1e-3, seed, stats=sa)
        rgc.rgc_apply_carried(wb, c, pg, 1e-3, seed, wn, fresh=fresh, stats=sb)
        torch.cuda.synchronize()
        s_a, s_b = sa.cpu().numpy()[2], sb.cpu().numpy()[2]
        ulps = abs(int(np.float32(s_a).view(np.int32)) - int(np.float32(s_b).view(np.int32)))
        assert ulps <= 1, (step, s_a, s_b)
        fresh = False
        if ulps == 0:
            assert np.array_equal(bits(wa), bits(wb)), f"step {step}"
        else:  # different s: restart the carried chain from the plain chain's weights
            wb.copy_(wa)
            fresh = True


@pytest.mark.parametrize("r", [64, 256])  # Gram-form norms; rebuilt norms and the scale launch
def test_carried_skip_keeps_weights_and_value(dev, r):
    d, k = 512, 1024
    w, p = _w_p(d, k, r, 8)
    wg = w.clone().to(dev)
    zero = torch.zeros(d, r, device=dev)
    wn = torch.full((1,), -7.0, dtype=torch.float64, device=dev)
    stats = torch.zeros(4, device=dev)
    # fresh: the streamed ||W||^2 is stored even though the update is skipped
    rgc.rgc_apply_carried(wg, zero, p.to(dev), 1e-3, 3, wn, fresh=True, stats=stats)
    torch.cuda.synchronize()
    assert np.array_equal(bits(wg), bits(w))
    assert stats.cpu().numpy()[3] == 1
    np.testing.assert_allclose(wn.item(), orc.weight_sumsq(bits(w)), rtol=1e-6)
    # carried: the caller's value is left bit for bit
    wn.fill_(12.375)
    rgc.rgc_apply_carried(wg, zero, p.to(dev), 1e-3, 3, wn, fresh=False, stats=stats)
    torch.cuda.synchronize()
    assert np.array_equal(bits(wg), bits(w))
    assert wn.item() == 12.375


def test_carried_batch_matches_single(dev):
    """A block-shaped batch (four shapes, one of them twice) against one call
    per matrix: the same weights bit for bit and the same carried values,
    over two steps (fresh, then carried); the values repeat on a rerun."""
    r = 64
    shapes = [(512, 256), (256, 256), (1536, 256), (256, 768), (512, 256)]
    Ws, Ps, Cs = [], [], []
    for i, (d, k) in enumerate(shapes):
        w, p = _w_p(d, k, r, 50 + i)
        Ws.append(w)
        Ps.append(p.to(dev))
    wb = [w.clone().to(dev) for w in Ws]
    ws = [w.clone().to(dev) for w in Ws]
    wnb = torch.zeros(len(shapes), dtype=torch.float64, device=dev)
    wns = [torch.zeros(1, dtype=torch.float64, device=dev) for _ in shapes]
    for step in range(2):
        Cs = [synth.normal_f32((d, r), 1e-2, seed=70 + 10 * step + i).to(dev) for i, (d, _) in enumerate(shapes)]
        seeds = [1000 + 17 * i + step for i in range(len(shapes))]
        rgc.rgc_apply_carried_batch(wb, Cs, Ps, 1e-3, seeds, wnb, fresh=(step == 0))
        for i in range(len(shapes)):
            rgc.rgc_apply_carried(ws[i], Cs[i], Ps[i], 1e-3, seeds[i], wns[i], fresh=(step == 0))
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert np.array_equal(bits(wb[i]), bits(ws[i])), f"step {step} item {i}"
            assert wnb[i].item() == wns[i].item(), f"step {step} item {i}"
    # determinism: the same call on the same inputs gives the same value
    again = [w.clone() for w in wb]
    v0 = torch.zeros(len(shapes), dtype=torch.float64, device=dev)
    v1 = torch.zeros(len(shapes), dtype=torch.float64, device=dev)
    rgc.rgc_apply_carried_batch(again, Cs, Ps, 1e-3, seeds, v0, fresh=True)
    again2 = [w.clone() for w in wb]
    rgc.rgc_apply_carried_batch(again2, Cs, Ps, 1e-3, seeds, v1, fresh=True)
    torch.cuda.synchronize()
    assert torch.equal(v0, v1)
    for a, b in zip(again, again2):
        assert torch.equal(a, b)
