"""Projects of matrices that read the same X in one pass over it.

A transformer block's q, k and v projections read one activation X, as do
gate and up; the layer keeps X P for each [page "Randomized Gradient
Compression", "How it works"]. rgc_project_shared projects up to four such
matrices as one stream-K item whose rank operand is their projections side
by side (up to 256 ranks), so each X slab is read once for all of them; the
batched project (rgc_project_batch) keeps one item per matrix whatever the
X pointers. Every XP must match the oracle's bf16(X P) to the project bar
(1 bf16 ulp + 2^-20 sum|x p|, at most 1e-3 of the elements differing).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_sum_close

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _check(xs, ps, outs, what):
    for i, (x, p, o) in enumerate(zip(xs, ps, outs)):
        xb, pb = bits(x), bits(p)
        abs_terms = np.abs(orc.bf16_to_f64(xb)) @ np.abs(orc.bf16_to_f64(pb))
        assert_sum_close(bits(o), orc.project(xb, pb), abs_terms, what=f"{what} item {i}")


# (T, k, r, members): 4 members (r = 16, 48 padded to 208, 64), 3 padded to
# 256 ranks (r = 80), 2 at r = 128, 1 at r = 256
@pytest.mark.parametrize("T,k,r,n", [(1000, 520, 64, 3), (300, 2048, 16, 4), (777, 1000, 48, 4), (513, 1048, 80, 3),
                                     (4096, 2048, 128, 2), (129, 264, 64, 4), (4096, 6144, 64, 2), (200, 520, 256, 1)])
def test_shared_x_members(dev, T, k, r, n):
    """n projections of one X (row stride k + 8) in one pass."""
    x_full = synth.normal_bf16((T, k + 8), 1.0, seed=r + n)
    x = x_full[:, :k]
    xg = x_full.to(dev)[:, :k]
    ps = [synth.normal_bf16((k, r), 1.0, seed=10 * r + i) for i in range(n)]
    outs = rgc.rgc_project_shared(xg, [p.to(dev) for p in ps])
    torch.cuda.synchronize()
    _check([x] * n, ps, outs, f"shared T={T} k={k} r={r} n={n}")


def test_block_projects_through_both_paths(dev):
    """A Qwen3-1.7B-shaped block's projections at r = 64, 4096 tokens: q, k, v
    and gate, up through rgc_project_shared, o and down through the batch; the
    same matrices through the batch alone give XP within the project bar."""
    T, r = 4096, 64
    xa, xo, xm = (synth.normal_bf16((T, 2048), 1.0, seed=50 + i) for i in range(3))
    xd = synth.normal_bf16((T, 6144), 1.0, seed=53)
    g = {n: t.to(dev) for n, t in (("a", xa), ("o", xo), ("m", xm), ("d", xd))}
    ps = [synth.normal_bf16((2048 if i < 6 else 6144, r), 1.0, seed=60 + i) for i in range(7)]
    pg = [p.to(dev) for p in ps]
    qkv = rgc.rgc_project_shared(g["a"], pg[0:3])
    gu = rgc.rgc_project_shared(g["m"], pg[4:6])
    od = rgc.rgc_project_batch([g["o"], g["d"]], [pg[3], pg[6]])
    batch = rgc.rgc_project_batch([g["a"], g["a"], g["a"], g["o"], g["m"], g["m"], g["d"]], pg)
    torch.cuda.synchronize()
    xs = [xa, xa, xa, xo, xm, xm, xd]
    _check(xs, ps, qkv[:3] + [od[0]] + gu + [od[1]], "shared + batch")
    _check(xs, ps, batch, "batch")


def test_shared_and_distinct_x_mixed(dev):
    """Two items on one X, one item on a copy of it (a different tensor: not
    grouped), two items on a third X; results match the oracle either way."""
    T, k, r = 640, 1024, 64
    x = synth.normal_bf16((T, k), 1.0, seed=5)
    y = synth.normal_bf16((T, k), 1.0, seed=6)
    xg, yg = x.to(dev), y.to(dev)
    xcopy = xg.clone()
    xs, xs_g = [x, x, x, y, y], [xg, xg, xcopy, yg, yg]
    ps = [synth.normal_bf16((k, r), 1.0, seed=20 + i) for i in range(5)]
    outs = rgc.rgc_project_batch(xs_g, [p.to(dev) for p in ps])
    torch.cuda.synchronize()
    _check(xs, ps, outs, "mixed")


@pytest.mark.parametrize("wgs", [1, 3, 7])
def test_shared_x_with_few_workgroups(dev, wgs):
    """Forced workgroup counts: ranges of whole group tiles, first segments
    kept past later ones, a K extent (72) with a partial step."""
    T, r = 300, 64
    for k, n, seed in ((520, 2, 7), (72, 3, 8)):
        x = synth.normal_bf16((T, k), 1.0, seed=seed)
        ps = [synth.normal_bf16((k, r), 1.0, seed=30 + i) for i in range(n)]
        outs = rgc.rgc_project_shared(x.to(dev), [p.to(dev) for p in ps], workgroups=wgs)
        torch.cuda.synchronize()
        _check([x] * n, ps, outs, f"wgs={wgs} k={k}")


def test_grouped_project_is_deterministic(dev):
    T, k, r = 4096, 2048, 64
    x = synth.normal_bf16((T, k), 1.0, seed=9).to(dev)
    ps = [synth.normal_bf16((k, r), 1.0, seed=40 + i).to(dev) for i in range(3)]
    a = [o.clone() for o in rgc.rgc_project_shared(x, ps)]
    b = rgc.rgc_project_shared(x, ps)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
