"""Pins for the oracle's random streams (CPU only).

Philox4x32-10 is checked against an independent implementation: ATen's
philox_engine header, compiled here with g++ (a library routine, not a copy).
The derived streams (signs, Gaussians, rounding bits) are checked in
distribution.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle as orc

TORCH_INCLUDE = None
try:
    import torch.utils.cpp_extension as _ce

    TORCH_INCLUDE = _ce.include_paths()[0]
except Exception:  # pragma: no cover
    pass

_ATEN_DRIVER = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
// Reads lines "c0 c1 c2 c3 k0 k1" (hex) and prints the four output words.
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (uint64_t(k1) << 32) | k0;
    uint64_t subseq = (uint64_t(c3) << 32) | c2;
    uint64_t offset = (uint64_t(c1) << 32) | c0;
    at::philox_engine e(seed, subseq, offset);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def aten_philox(tmp_path_factory):
    if TORCH_INCLUDE is None or shutil.which("g++") is None:
        pytest.skip("g++ or torch headers unavailable")
    d = tmp_path_factory.mktemp("aten_philox")
    src = d / "kat.cpp"
    src.write_text(_ATEN_DRIVER)
    exe = d / "kat"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", TORCH_INCLUDE, str(src), "-o", str(exe)], check=True)
    return str(exe)


def test_philox_matches_aten_engine(aten_philox):
    rng = np.random.default_rng(1234)
    n = 2000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    # include the all-zero and all-ones corners
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 2**32 - 1
    key[1] = 2**32 - 1
    lines = "\n".join(" ".join(f"{int(v):x}" for v in list(c) + list(k)) for c, k in zip(ctr, key))
    out = subprocess.run([aten_philox], input=lines, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(t, 16) for t in ln.split()] for ln in out.strip().splitlines()], dtype=np.uint64)
    got = np.stack(orc.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], key[:, 0], key[:, 1]), axis=1)
    assert got.shape == ref.shape
    assert np.array_equal(got.astype(np.uint64), ref)


def test_rounding_bits_uniform_and_uncorrelated():
    """16-bit rounding draws: chi-square over 2^16 bins; adjacent rows/cols uncorrelated."""
    r16 = orc.rounding_bits(seed=0xC0FFEE, rows=1024, cols=4096).astype(np.int64)
    counts = np.bincount(r16.ravel(), minlength=1 << 16)
    chi2 = float(((counts - counts.mean()) ** 2 / counts.mean()).sum())
    p = stats.chi2.sf(chi2, df=(1 << 16) - 1)
    assert p > 1e-3, p
    u = r16.astype(np.float64) / 65536.0 - 0.5
    for a, b in ((u[:, 1:], u[:, :-1]), (u[1:, :], u[:-1, :])):
        corr = float(np.mean(a * b) / np.mean(u * u))
        assert abs(corr) < 5.0 / np.sqrt(a.size), corr


def test_rounding_bits_offsets_are_consistent():
    """A sub-block drawn with (row0, col0) equals the same block of the full draw."""
    full = orc.rounding_bits(7, 40, 70)
    sub = orc.rounding_bits(7, 13, 29, row0=11, col0=21)
    assert np.array_equal(full[11:24, 21:50], sub)


def test_rademacher_entries_and_balance():
    k, r = 4096, 256
    p = orc.rademacher_projection(42, k, r)
    vals = orc.bf16_to_f64(p)
    assert set(np.unique(np.abs(vals))) == {1.0 / 16.0}
    neg = np.count_nonzero(vals < 0)
    # binomial(k*r, 1/2): within 5 sigma
    n = k * r
    assert abs(neg - n / 2) < 5 * np.sqrt(n / 4)
    # P^T P diagonal is exactly k/r (each entry squared is 1/r)
    gram = vals.T @ vals
    assert np.array_equal(np.diag(gram), np.full(r, k / r))
    off = gram[~np.eye(r, dtype=bool)]
    # off-diagonals: (1/r) times a sum of k independent signs -> variance k/r^2
    assert abs(off.mean()) < 5 * np.sqrt(k) / r / np.sqrt(off.size / 2)
    assert abs(off.var() / (k / r**2) - 1.0) < 0.05


def test_rademacher_seeds_differ_and_repeat():
    a = orc.rademacher_projection(1, 64, 32)
    b = orc.rademacher_projection(1, 64, 32)
    c = orc.rademacher_projection(2, 64, 32)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_gaussian_is_standard_normal():
    z = orc.gaussian_matrix(99, 2048, 64).ravel()
    ks = stats.kstest(z, "norm")
    assert ks.pvalue > 1e-3, ks
    assert abs(z.mean()) < 5 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / z.size)
    # the cos/sin partners of one Box-Muller pair are uncorrelated
    zz = orc.gaussian_matrix(5, 4096, 64)
    c = np.corrcoef(zz[:, 0::2].ravel(), zz[:, 1::2].ravel())[0, 1]
    assert abs(c) < 5 / np.sqrt(zz.size / 2)


def test_gaussian_batched_equals_single():
    seeds = np.array([3, 17, 2**40 + 5], dtype=np.uint64)
    zb = orc.gaussian_matrix(seeds, 24, 16)
    for s, z in zip(seeds, zb):
        assert np.array_equal(z, orc.gaussian_matrix(int(s), 24, 16))
