"""The deferred accumulation (rgc_accumulate_batch_deferred): the microbatches
of one accumulation add into the same sketches [RGC, "How it works"; LoGRA-S,
Key Contributions 1], with the split tiles' partial sums kept in the
workspace between the calls and added into C once, by the last call.

Against the oracle's per-microbatch loop (C rounded to fp32 after every
microbatch): relative Frobenius error below 1e-5 after the last call, at
every kind of rank (4 and 8: small-rank kernels, which finish every call;
tiled ranks, split tiles present), with ranges forced across items and tile
ends, and bit-identical when repeated. A single call with both phase bits is
rgc_accumulate_batch itself, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _inputs(T, ds, r, n_mb, seed):
    dd = [[synth.normal_bf16((T, d), 1e-3, seed=seed + 100 * i + m) for m, d in enumerate(ds)] for i in range(n_mb)]
    xp = [[synth.normal_bf16((T, r), 3.0, seed=seed + 100 * i + 50 + m) for m in range(len(ds))] for i in range(n_mb)]
    c0 = [synth.normal_f32((d, r), 1e-3, seed=seed + 7000 + m) for m, d in enumerate(ds)]
    return dd, xp, c0


def _oracle(dd, xp, c0):
    cs = [c.numpy().copy() for c in c0]
    for i in range(len(dd)):
        cs = [orc.accumulate(cs[m], bits(dd[i][m]), bits(xp[i][m])) for m in range(len(cs))]
    return cs


def _run(dev, dd, xp, c0, workgroups=0):
    cs = [c.clone().to(dev) for c in c0]
    ws = rgc.Workspace(dev)
    n_mb = len(dd)
    for i in range(n_mb):
        rgc.rgc_accumulate_batch_deferred([d.to(dev) for d in dd[i]], [x.to(dev) for x in xp[i]], cs, ws,
                                          first=(i == 0), last=(i == n_mb - 1), workgroups=workgroups)
    torch.cuda.synchronize()
    return cs


@pytest.mark.parametrize("r", [4, 8, 64, 128, 256])
def test_deferred_matches_oracle(dev, r):
    T, ds, n_mb = 1000, [520, 1048, 264], 5
    dd, xp, c0 = _inputs(T, ds, r, n_mb, seed=r)
    got = _run(dev, dd, xp, c0)
    for g, ref in zip(got, _oracle(dd, xp, c0)):
        assert rel_frobenius(g.cpu().numpy(), ref) < 1e-5


@pytest.mark.parametrize("wgs", [1, 3, 7, 64])
def test_deferred_forced_workgroups(dev, wgs):
    """Ranges that cover whole tiles, cross item boundaries, or cut every tile."""
    T, ds, r, n_mb = 300, [264, 520], 64, 3
    dd, xp, c0 = _inputs(T, ds, r, n_mb, seed=90 + wgs)
    got = _run(dev, dd, xp, c0, workgroups=wgs)
    for g, ref in zip(got, _oracle(dd, xp, c0)):
        assert rel_frobenius(g.cpu().numpy(), ref) < 1e-5


def test_single_call_is_the_plain_batch(dev):
    T, ds, r = 4096, [2048, 1024, 6144], 64
    dd, xp, c0 = _inputs(T, ds, r, 1, seed=5)
    a = [c.clone().to(dev) for c in c0]
    b = [c.clone().to(dev) for c in c0]
    D = [d.to(dev) for d in dd[0]]
    X = [x.to(dev) for x in xp[0]]
    rgc.rgc_accumulate_batch(D, X, a)
    rgc.rgc_accumulate_batch_deferred(D, X, b, rgc.Workspace(dev), first=True, last=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_deferred_full_size_block_is_deterministic(dev):
    """The 8 x 4096-token accumulation of a Qwen3-1.7B-shaped block's seven
    matrices at r = 64, twice: the same bits; against the oracle's loop."""
    T, ds, r, n_mb = 4096, [2048, 1024, 1024, 2048, 6144, 6144, 2048], 64, 8
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    D = [[(torch.randn(T, d, generator=g, device=dev) * 1e-3).to(torch.bfloat16) for d in ds] for _ in range(n_mb)]
    X = [[(torch.randn(T, r, generator=g, device=dev) * 3).to(torch.bfloat16) for _ in ds] for _ in range(n_mb)]
    runs = []
    for _ in range(2):
        cs = [torch.zeros(d, r, device=dev) for d in ds]
        ws = rgc.Workspace(dev)
        for i in range(n_mb):
            rgc.rgc_accumulate_batch_deferred(D[i], X[i], cs, ws, first=(i == 0), last=(i == n_mb - 1))
        torch.cuda.synchronize()
        runs.append(cs)
    for u, v in zip(*runs):
        assert torch.equal(u, v)
    ref = [np.zeros((d, r), np.float32) for d in ds]
    for i in range(n_mb):
        ref = [orc.accumulate(ref[m], bits(D[i][m]), bits(X[i][m])) for m in range(len(ds))]
    for u, c in zip(runs[0], ref):
        assert rel_frobenius(u.cpu().numpy(), c) < 1e-5
