"""The layer's own products on the library's kernels: rgc_linear_forward
([Y | XP] = X [W^T | P], one tile grid) and rgc_linear_backward (dX = D W,
then C += D^T XP) [RGC, "How it works"; LoGRA-M, "Minimal Causal Code"].

Against the oracle's layer_forward / layer_backward on the same seeded bits:
Y, XP and dX within one bf16 ulp plus 2^-20 sum|ab| (the fp32 summation
error of a long sum; at most 1e-3 of the elements differing), C within 1e-5
relative Frobenius and bit-identical to rgc_accumulate's. Y and dX are also
checked against an fp32 torch reference (relative Frobenius < 4e-3, the
bf16 output rounding). Shapes are ragged in every dimension: T, d, k not
multiples of the 256 x 256 tile or of the 32-row K-step, K below one step,
a single token row, strided X, Y and dX; every rank through the forward
(XP as slices inside Y's tiles, or as a column of tiles of its own).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_sum_close, rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _absprod(a_bits, b_bits):
    return np.abs(orc.bf16_to_f64(a_bits)) @ np.abs(orc.bf16_to_f64(b_bits))


def _fp32_ref(a, b):
    return (a.float() @ b.float()).numpy()


# (T, k, d, r): tile tails in T and d, K tails (72 = two steps + 8, 40 = one
# step + 8, 1000), r = 0 (Y alone), 4 (XP from the small-rank project), 8 (a
# P narrower than a block: a column of tiles), up to 256
SHAPES = [(300, 520, 264, 64), (256, 512, 512, 128), (77, 1000, 1048, 16), (513, 72, 136, 8),
          (1000, 2048, 520, 256), (1, 40, 8, 32), (129, 264, 776, 0), (600, 1048, 200, 4),
          (257, 64, 264, 48), (4096, 1024, 1024, 128)]


@pytest.mark.parametrize("T,k,d,r", SHAPES)
def test_forward_matches_oracle(dev, T, k, d, r):
    x = synth.normal_bf16((T, k), 1.0, seed=T + k)
    w = synth.normal_bf16((d, k), 0.02, seed=d + 1)
    p = synth.normal_bf16((k, r), 1.0, seed=r + 2) if r else None
    y, xp = rgc.rgc_linear_forward(x.to(dev), w.to(dev), p.to(dev) if p is not None else None)
    torch.cuda.synchronize()
    y_ref, xp_ref = orc.layer_forward(bits(x), bits(w), bits(p) if p is not None else None)
    assert_sum_close(bits(y), y_ref, _absprod(bits(x), bits(w).T), what=f"Y T={T} k={k} d={d}")
    assert rel_frobenius(y.float().cpu().numpy(), _fp32_ref(x, w.T)) < 4e-3
    if r:
        assert_sum_close(bits(xp), xp_ref, _absprod(bits(x), bits(p)), what=f"XP r={r}")
    else:
        assert xp is None


@pytest.mark.parametrize("T,k,d,r", SHAPES)
def test_backward_matches_oracle(dev, T, k, d, r):
    dd = synth.normal_bf16((T, d), 1e-3, seed=T + d + 3)
    w = synth.normal_bf16((d, k), 0.02, seed=k + 4)
    xp = synth.normal_bf16((T, r), 3.0, seed=r + 5) if r else None
    c0 = synth.normal_f32((d, r), 1e-3, seed=r + 6) if r else None
    c = c0.clone().to(dev) if r else None
    c_acc = c0.clone().to(dev) if r else None
    dg = dd.to(dev)
    dx = rgc.rgc_linear_backward(dg, w.to(dev), xp.to(dev) if r else None, c)
    if r:
        rgc.rgc_accumulate(dg, xp.to(dev), c_acc)
    torch.cuda.synchronize()
    dx_ref, c_ref = orc.layer_backward(bits(dd), bits(w), bits(xp) if r else None, c0.numpy() if r else None)
    assert_sum_close(bits(dx), dx_ref, _absprod(bits(dd), bits(w)), what=f"dX T={T} k={k} d={d}")
    assert rel_frobenius(dx.float().cpu().numpy(), _fp32_ref(dd, w)) < 4e-3
    if r:
        assert rel_frobenius(c.cpu().numpy(), c_ref) < 1e-5
        assert torch.equal(c, c_acc)  # the same accumulate, the same bits


def test_strided_operands(dev):
    """X, Y and dX as column windows of wider buffers (row strides k + 24,
    d + 40, k + 8); the bytes around the windows stay untouched."""
    T, k, d, r = 333, 520, 264, 32
    xf = synth.normal_bf16((T, k + 24), 1.0, seed=1)
    w = synth.normal_bf16((d, k), 0.02, seed=2)
    p = synth.normal_bf16((k, r), 1.0, seed=3)
    xg = xf.to(dev)[:, 8:8 + k]
    yfull = torch.full((T, d + 40), 7.0, dtype=torch.bfloat16, device=dev)
    y = yfull[:, 16:16 + d]
    _, xp = rgc.rgc_linear_forward(xg, w.to(dev), p.to(dev), Y=y)
    dd = synth.normal_bf16((T, d), 1e-3, seed=4)
    dxfull = torch.full((T, k + 8), 5.0, dtype=torch.bfloat16, device=dev)
    rgc.rgc_linear_backward(dd.to(dev), w.to(dev), dX=dxfull[:, :k])
    torch.cuda.synchronize()
    x = xf[:, 8:8 + k].contiguous()
    y_ref, xp_ref = orc.layer_forward(bits(x), bits(w), bits(p))
    assert_sum_close(bits(y), y_ref, _absprod(bits(x), bits(w).T), what="strided Y")
    assert_sum_close(bits(xp), xp_ref, _absprod(bits(x), bits(p)), what="strided XP")
    assert bool((yfull[:, :16] == 7).all()) and bool((yfull[:, 16 + d:] == 7).all())
    dx_ref, _ = orc.layer_backward(bits(dd), bits(w), None, None)
    assert_sum_close(bits(dxfull[:, :k]), dx_ref, _absprod(bits(dd), bits(w)), what="strided dX")
    assert bool((dxfull[:, k:] == 5).all())


def test_forward_batch_shared_input(dev):
    """A block's q, k, v (one X, d = 512, 128, 128) and gate (another X) in one
    launch; each item as the single call gives it, bit for bit."""
    T, k, r = 700, 512, 64
    xa = synth.normal_bf16((T, k), 1.0, seed=20).to(dev)
    xb = synth.normal_bf16((T, k), 1.0, seed=21).to(dev)
    ws = [synth.normal_bf16((dm, k), 0.02, seed=22 + i).to(dev) for i, dm in enumerate((512, 128, 128, 1000))]
    ps = [synth.normal_bf16((k, r), 1.0, seed=30 + i).to(dev) for i in range(4)]
    xs = [xa, xa, xa, xb]
    ys, xps = rgc.rgc_linear_forward_batch(xs, ws, ps)
    single = [rgc.rgc_linear_forward(x, w, p) for x, w, p in zip(xs, ws, ps)]
    torch.cuda.synchronize()
    for (y1, xp1), y, xp in zip(single, ys, xps):
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
        assert torch.equal(xp.view(torch.int16), xp1.view(torch.int16))
    y_ref, xp_ref = orc.layer_forward(bits(xb), bits(ws[3]), bits(ps[3]))
    assert_sum_close(bits(ys[3]), y_ref, _absprod(bits(xb), bits(ws[3]).T), what="batch gate Y")


def test_forward_and_backward_are_deterministic(dev):
    T, k, d, r = 1000, 1048, 776, 128
    x = synth.normal_bf16((T, k), 1.0, seed=40).to(dev)
    w = synth.normal_bf16((d, k), 0.02, seed=41).to(dev)
    p = synth.normal_bf16((k, r), 1.0, seed=42).to(dev)
    dd = synth.normal_bf16((T, d), 1e-3, seed=43).to(dev)
    a = [t.clone() for t in rgc.rgc_linear_forward(x, w, p)] + [rgc.rgc_linear_backward(dd, w).clone()]
    b = list(rgc.rgc_linear_forward(x, w, p)) + [rgc.rgc_linear_backward(dd, w)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


def test_qwen3_8b_gate_shape_sampled_rows(dev):
    """The 8B MLP gate layer at full size (4096 tokens, k = 4096, d = 12288,
    r = 128): 48 sampled token rows of Y, XP and dX against the oracle (each
    row is an independent sum), C against the accumulate."""
    T, k, d, r = 4096, 4096, 12288, 128
    xg = synth.normal_bf16((T, k), 1.0, seed=50, device=dev)
    wg = synth.normal_bf16((d, k), 0.02, seed=51, device=dev)
    pg = synth.normal_bf16((k, r), 1.0 / np.sqrt(r), seed=52, device=dev)
    dg = synth.normal_bf16((T, d), 1e-3, seed=53, device=dev)
    y, xp = rgc.rgc_linear_forward(xg, wg, pg)
    c = torch.zeros(d, r, device=dev)
    c_acc = torch.zeros(d, r, device=dev)
    dx = rgc.rgc_linear_backward(dg, wg, xp, c)
    rgc.rgc_accumulate(dg, xp, c_acc)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(T, 48, replace=False)
    rows[:2] = [0, T - 1]
    sel = torch.as_tensor(rows, device=dev)
    x, w, p, dd = bits(xg[sel]), bits(wg), bits(pg), bits(dg[sel])
    y_ref, xp_ref = orc.layer_forward(x, w, p)
    assert_sum_close(bits(y[sel]), y_ref, _absprod(x, w.T), what="8B gate Y rows")
    assert_sum_close(bits(xp[sel]), xp_ref, _absprod(x, p), what="8B gate XP rows")
    dx_ref, _ = orc.layer_backward(dd, w, None, None)
    assert_sum_close(bits(dx[sel]), dx_ref, _absprod(dd, w), what="8B gate dX rows")
    assert torch.equal(c, c_acc)


def test_rejects_bad_arguments(dev):
    x = torch.zeros(16, 64, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(32, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(rgc.RgcError):  # k not a multiple of 8
        rgc.rgc_linear_forward(x[:, :60], w[:, :60])
    with pytest.raises(rgc.RgcError):  # unsupported rank
        rgc.rgc_linear_forward(x, w, torch.zeros(64, 24, dtype=torch.bfloat16, device=dev))
    with pytest.raises(rgc.RgcError):  # rank above k
        rgc.rgc_linear_forward(x[:, :16], w[:, :16], torch.zeros(16, 32, dtype=torch.bfloat16, device=dev))
    with pytest.raises(rgc.RgcError):  # XP without C
        rgc.rgc_linear_backward(torch.zeros(16, 32, dtype=torch.bfloat16, device=dev), w,
                                XP=torch.zeros(16, 16, dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("r", [16 * q for q in range(1, 17)])
@pytest.mark.parametrize("d", [264, 1048])
def test_forward_every_rank(dev, d, r):
    """Every tiled rank through the forward, at two widths of Y: XP as slices
    inside Y's tiles where a tile carries at most two (r <= 64 at d = 264,
    r <= 160 at d = 1048), else as one more column of tiles."""
    T, k = 300, 520
    x = synth.normal_bf16((T, k), 1.0, seed=r + d)
    w = synth.normal_bf16((d, k), 0.02, seed=r + d + 1)
    p = synth.normal_bf16((k, r), 1.0, seed=r + d + 2)
    y, xp = rgc.rgc_linear_forward(x.to(dev), w.to(dev), p.to(dev))
    torch.cuda.synchronize()
    y_ref, xp_ref = orc.layer_forward(bits(x), bits(w), bits(p))
    assert_sum_close(bits(y), y_ref, _absprod(bits(x), bits(w).T), what=f"Y d={d} r={r}")
    assert_sum_close(bits(xp), xp_ref, _absprod(bits(x), bits(p)), what=f"XP d={d} r={r}")
