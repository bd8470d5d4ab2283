"""The sketched linear layer: forward keeps X P instead of X, backward adds
D^T (X P) to the sketch and passes D W on, the update matches the oracle's
(the small single-layer case: d = 256, k = 512, r = 16, 4 x 256 tokens)."""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import SketchedLinear, rgc, synth
from parity_tools import assert_sum_close, assert_update_close, qr_margin_mismatches, rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


@pytest.mark.parametrize("mode", ["normalized", "scaled"])
def test_sketched_linear_training_step(dev, mode):
    d, k, r, mb, n_mb, seed = 256, 512, 16, 256, 4, 0
    x = synth.normal_bf16((mb * n_mb, k), 1.0, seed=1000)
    dd = synth.normal_bf16((mb * n_mb, d), 0.1, seed=1001)
    w = synth.normal_bf16((d, k), 0.02, seed=1002)
    layer = SketchedLinear(k, d, r, kind="qr", device=dev, weight=w.clone())
    layer.begin_update(seed)
    xg, dg = x.to(dev), dd.to(dev)
    for i in range(n_mb):
        xi = xg[i * mb:(i + 1) * mb].view(2, mb // 2, k).clone().requires_grad_(True)  # a (batch, seq, k) input
        y = layer(xi)
        assert y.shape == (2, mb // 2, d)
        # the layer keeps X P (tokens x r), never X (tokens x k)
        saved = y.grad_fn.saved_tensors
        assert all(t.shape[-1] != k or t.shape[0] == d for t in saved)
        assert any(tuple(t.shape) == (mb, r) for t in saved)
        dyi = dg[i * mb:(i + 1) * mb].view(2, mb // 2, d)
        y.backward(dyi)
        # input gradient D W against an fp32 reference on the CPU
        ref_dx = dyi.float().cpu().reshape(mb, d) @ w.float()
        got_dx = xi.grad.float().cpu().reshape(mb, k)
        assert rel_frobenius(got_dx.numpy(), ref_dx.numpy()) < 1e-2
    assert layer.weight.grad is None
    torch.cuda.synchronize()
    # C and P against the oracle's loop
    p_ref = orc.qr_projection(seed, k, r)
    assert np.array_equal(bits(layer.proj), p_ref)
    c_ref = np.zeros((d, r), dtype=np.float32)
    for i in range(n_mb):
        c_ref = orc.accumulate(c_ref, bits(dd[i * mb:(i + 1) * mb]), orc.project(bits(x[i * mb:(i + 1) * mb]), p_ref))
    c = layer.sketch.cpu().numpy()
    assert rel_frobenius(c, c_ref) < 2e-3
    abs_terms = np.abs(c.astype(np.float64)) @ np.abs(orc.bf16_to_f64(p_ref)).T
    if mode == "normalized":
        stats = torch.zeros(4, device=dev)
        layer.apply_update(seed, tau=1e-3, stats=stats)
        torch.cuda.synchronize()
        ref_w, ref_stats = orc.apply_update(bits(w), c, p_ref, 1e-3, seed)
        s = ref_stats[2]
        np.testing.assert_allclose(stats.cpu().numpy()[:3], ref_stats[:3], rtol=1e-5)
    else:
        # a step of the size the normalized update takes here (s ~ 1e-6 for this
        # sketch): the update then moves each weight by a small fraction of itself
        s = np.float32(2e-6)
        layer.apply_update(seed, alpha=float(s))
        torch.cuda.synchronize()
        ref_w = orc.apply_scaled(bits(w), c, p_ref, s, seed)
    assert_update_close(bits(layer.weight.data), ref_w, s, abs_terms, what=f"layer update ({mode})")


def test_sketched_linear_requires_a_projection(dev):
    layer = SketchedLinear(512, 256, 16, device=dev)
    with pytest.raises(rgc.RgcError):
        layer(torch.zeros(4, 512, dtype=torch.bfloat16, device=dev))
    with pytest.raises(rgc.RgcError):
        layer.apply_update(0, tau=1e-3, alpha=1e-3)


def test_sketched_linear_carried_norm_matches_plain(dev):
    """Two layers on the same inputs over four updates, one carrying ||W||
    between its normalized updates (with a fixed-step update in between,
    after which the norm is streamed again): the same step s up to its last
    bit, and with an equal s the same weights."""
    d, k, r, mb = 512, 1024, 64, 512
    w = synth.normal_bf16((d, k), 0.02, seed=2002)
    plain = SketchedLinear(k, d, r, kind="qr", device=dev, weight=w.clone())
    carry = SketchedLinear(k, d, r, kind="qr", device=dev, weight=w.clone(), carry_norm=True)
    for u, how in enumerate(["tau", "tau", "alpha", "tau"]):
        x = synth.normal_bf16((mb, k), 1.0, seed=2100 + u).to(dev).requires_grad_(True)
        dy = synth.normal_bf16((mb, d), 0.1, seed=2200 + u).to(dev)
        stats = []
        for layer in (plain, carry):
            layer.begin_update(300 + u)
            layer(x).backward(dy)
            st = torch.zeros(4, device=dev)
            if how == "tau":
                layer.apply_update(400 + u, tau=1e-3, stats=st)
            else:
                layer.apply_update(400 + u, alpha=2e-6)
            stats.append(st)
        torch.cuda.synchronize()
        if how == "tau":
            sa, sb = (np.float32(s.cpu().numpy()[2]) for s in stats)
            assert sa > 0
            ulps = abs(int(sa.view(np.int32)) - int(sb.view(np.int32)))
            assert ulps <= 1, (u, sa, sb)
            if ulps:
                carry.weight.data.copy_(plain.weight.data)
                carry.invalidate_weight_norm()
                continue
        assert torch.equal(plain.weight.data, carry.weight.data), f"update {u}"


@pytest.mark.parametrize("how", ["copy", "load_state_dict"])
def test_sketched_linear_carried_norm_sees_weight_changes(dev, how):
    """Weights replaced between carried updates through the Parameter (an
    in-place copy, or load_state_dict): the next update streams ||W|| again
    without an explicit invalidate_weight_norm(), so it equals the plain
    layer's update bit for bit (same ||W||, same s, same weights)."""
    d, k, r, mb = 256, 512, 16, 256
    w = synth.normal_bf16((d, k), 0.02, seed=3002)
    w2 = synth.normal_bf16((d, k), 0.05, seed=3003).to(dev)
    plain = SketchedLinear(k, d, r, kind="qr", device=dev, weight=w.clone())
    carry = SketchedLinear(k, d, r, kind="qr", device=dev, weight=w.clone(), carry_norm=True)
    for u in range(2):
        x = synth.normal_bf16((mb, k), 1.0, seed=3100 + u).to(dev).requires_grad_(True)
        dy = synth.normal_bf16((mb, d), 0.1, seed=3200 + u).to(dev)
        stats = []
        for layer in (plain, carry):
            layer.begin_update(500 + u)
            layer(x).backward(dy)
            st = torch.zeros(4, device=dev)
            layer.apply_update(600 + u, tau=1e-3, stats=st)
            stats.append(st)
        torch.cuda.synchronize()
        if u == 1:
            assert torch.equal(stats[0], stats[1])
            assert torch.equal(plain.weight.data, carry.weight.data)
        # replace both layers' weights by the same new values
        with torch.no_grad():
            plain.weight.copy_(w2)
        if how == "copy":
            with torch.no_grad():
                carry.weight.copy_(w2)
        else:
            sd = carry.state_dict()
            sd["weight"] = w2.clone()
            sd["weight_norm2"] = torch.zeros(1, dtype=torch.float64, device=dev)  # a norm that does not match
            carry.load_state_dict(sd)


@pytest.mark.parametrize("r,kind", [(4, "rademacher"), (8, "qr"), (64, "qr")])
def test_sketched_linear_every_forward_path(dev, r, kind):
    """The layer at r = 4 (XP from the small-rank project after the tile
    grid), r = 8 (XP as one more column of tiles) and r = 64 (XP as slices
    inside Y's tiles): Y and dX against the oracle's layer products, the
    sketch against the oracle's loop, the saved tensors XP and W only."""
    d, k, mb, n_mb, seed = 264, 520, 300, 2, 7
    w = synth.normal_bf16((d, k), 0.02, seed=4000 + r)
    layer = SketchedLinear(k, d, r, kind=kind, device=dev, weight=w.clone())
    layer.begin_update(seed)
    p_ref = orc.sample_projection(kind, seed, k, r)
    c_ref = np.zeros((d, r), np.float32)
    for i in range(n_mb):
        x = synth.normal_bf16((mb, k), 1.0, seed=4100 + 10 * r + i)
        dy = synth.normal_bf16((mb, d), 0.1, seed=4200 + 10 * r + i)
        xg = x.to(dev).requires_grad_(True)
        y = layer(xg)
        assert sorted(tuple(t.shape) for t in y.grad_fn.saved_tensors) == sorted([(mb, r), (d, k)])
        y.backward(dy.to(dev))
        torch.cuda.synchronize()
        y_ref, xp_ref = orc.layer_forward(bits(x), bits(w), p_ref)
        absy = np.abs(orc.bf16_to_f64(bits(x))) @ np.abs(orc.bf16_to_f64(bits(w))).T
        assert_sum_close(bits(y.detach()), y_ref, absy, what=f"Y r={r}")
        dx_ref, c_ref = orc.layer_backward(bits(dy), bits(w), xp_ref, c_ref)
        absd = np.abs(orc.bf16_to_f64(bits(dy))) @ np.abs(orc.bf16_to_f64(bits(w)))
        assert_sum_close(bits(xg.grad), dx_ref, absd, what=f"dX r={r}")
    if kind == "rademacher":
        assert np.array_equal(bits(layer.proj), p_ref)
    else:
        assert qr_margin_mismatches(bits(layer.proj), seed, k, r) <= 2
    assert rel_frobenius(layer.sketch.cpu().numpy(), c_ref) < 1e-4
