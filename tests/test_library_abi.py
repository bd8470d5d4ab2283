"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before launching anything (CPU only: no call here ever
reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import rank_randomized_gradient_amd as rgc_pkg
from rank_randomized_gradient_amd import rgc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rgc.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, VALUE = 0, 1, 2, 3, 4, 5, 7
FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rgc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rgc.LIB_PATH):
        pytest.fail("librgc.so is not built (run __graft_entry__.build())")
    return rgc.load_library()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(rgc.SIGNATURES), set(names) ^ set(rgc.SIGNATURES)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define RGC_ABI_VERSION (\d+)", open(HEADER).read())
    assert rgc_pkg.abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(9):
        assert b"unknown" not in lib.rgc_status_string(s)
    assert b"unknown" in lib.rgc_status_string(99)


def test_workspace_queries(lib):
    assert lib.rgc_sample_projection_workspace_size(0, 2048, 64) == 0
    qr = lib.rgc_sample_projection_workspace_size(1, 2048, 64)
    # r >= 16: the Gaussian (k x r fp64), the summed Gram, one partial Gram per workgroup of 192 rows,
    # U1, U2 and flags; Q1 is formed again where it is needed rather than stored
    assert 2048 * 64 * 8 + (2048 + 191) // 192 * 64 * 64 * 8 + 3 * 64 * 64 * 8 <= qr < 2 * 2048 * 64 * 8
    # r = 4, 8: one partial per 64-row block, and the Gaussian and Q1 kept (k x r fp64 each)
    assert lib.rgc_sample_projection_workspace_size(1, 2048, 8) >= 2 * 2048 * 8 * 8 + 2048 // 64 * 8 * 8 * 8
    assert lib.rgc_sample_projection_workspace_size(1, 2048, 256) == 0  # QR limited to r <= 128
    assert lib.rgc_accumulate_workspace_size(4096, 2048, 64) >= 0
    small = lib.rgc_apply_workspace_size(2048, 2048, 64)  # per-workgroup norm partials + step scalars
    assert small > 0 and lib.rgc_apply_workspace_size(8192, 8192, 64) > small
    assert lib.rgc_apply_workspace_size(2048, 2048, 40) == 0  # unsupported rank


def test_project_validation(lib):
    s = None
    # shape errors
    assert lib.rgc_project(FAKE, 63, FAKE, FAKE, 16, 64, 16, None, 0, s) == SHAPE  # ldx < k
    assert lib.rgc_project(FAKE, 64, FAKE, FAKE, -1, 64, 16, None, 0, s) == SHAPE
    assert lib.rgc_project(FAKE, 64, FAKE, FAKE, 16, 8, 16, None, 0, s) == SHAPE  # r > k
    # unsupported
    assert lib.rgc_project(FAKE, 64, FAKE, FAKE, 16, 64, 24, None, 0, s) == UNSUP
    assert lib.rgc_project(FAKE, 68, FAKE, FAKE, 16, 68, 16, None, 0, s) == UNSUP  # k % 8
    # T = 0 is a no-op
    assert lib.rgc_project(None, 64, None, None, 0, 64, 16, None, 0, s) == OK
    assert lib.rgc_project(None, 64, FAKE, FAKE, 16, 64, 16, None, 0, s) == NULL
    assert lib.rgc_project(FAKE + 2, 64, FAKE, FAKE, 16, 64, 16, None, 0, s) == ALIGN
    assert lib.rgc_project(FAKE, 68, FAKE, FAKE, 16, 64, 16, None, 0, s) == ALIGN  # ldx % 8
    need = lib.rgc_project_workspace_size(4096, 2048, 64)
    assert need > 0
    assert lib.rgc_project(FAKE, 2048, FAKE, FAKE, 4096, 2048, 64, None, 0, s) == WS
    assert lib.rgc_project(FAKE, 2048, FAKE, FAKE, 4096, 2048, 64, FAKE, need - 1, s) == WS
    assert lib.rgc_project(FAKE, 2048, FAKE, FAKE, 4096, 2048, 64, FAKE + 16, need, s) == ALIGN
    assert lib.rgc_project(FAKE, (1 << 23) + 8, FAKE, FAKE, 16, 64, 16, None, 0, s) == UNSUP  # ldx > 2^23


def test_accumulate_validation(lib):
    s = None
    assert lib.rgc_accumulate(FAKE, 255, FAKE, FAKE, 16, 256, 16, None, 0, s) == SHAPE
    assert lib.rgc_accumulate(FAKE, 256, FAKE, FAKE, 16, 256, 20, None, 0, s) == UNSUP
    assert lib.rgc_accumulate(FAKE, 260, FAKE, FAKE, 16, 260, 16, None, 0, s) == UNSUP
    assert lib.rgc_accumulate(None, 256, None, None, 0, 256, 16, None, 0, s) == OK
    assert lib.rgc_accumulate(FAKE, 256, None, FAKE, 16, 256, 16, None, 0, s) == NULL
    assert lib.rgc_accumulate(FAKE, 256, FAKE, FAKE + 4, 16, 256, 16, None, 0, s) == ALIGN
    need = lib.rgc_accumulate_workspace_size(4096, 2048, 64)
    assert need > 0
    assert lib.rgc_accumulate(FAKE, 2048, FAKE, FAKE, 4096, 2048, 64, FAKE, need - 4, s) == WS
    assert lib.rgc_accumulate(FAKE, 1 << 20, FAKE, FAKE, 4096, 1 << 20, 64, FAKE, need, s) == UNSUP  # d > limit
    assert lib.rgc_accumulate(FAKE, (1 << 23) + 8, FAKE, FAKE, 16, 256, 16, None, 0, s) == UNSUP  # ldd > 2^23


def test_apply_validation(lib):
    s = None
    f = ctypes.c_float(1e-3)
    assert lib.rgc_apply(FAKE, 255, FAKE, FAKE, 64, 256, 16, f, 0, None, FAKE, 1 << 20, s) == SHAPE
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 64, 256, 272, f, 0, None, FAKE, 1 << 20, s) == SHAPE  # r > k
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 60, 256, 16, f, 0, None, FAKE, 1 << 20, s) == UNSUP
    assert lib.rgc_apply(FAKE, 256, None, FAKE, 64, 256, 16, f, 0, None, FAKE, 1 << 20, s) == NULL
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 64, 256, 16, f, 0, FAKE + 2, FAKE, 1 << 20, s) == ALIGN
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 64, 256, 16, f, 0, None, None, 0, s) == WS
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 64, 256, 16, f, 0, None, FAKE + 64, 1 << 20, s) == ALIGN


def test_apply_batch_validation(lib):
    s = None
    f = ctypes.c_float(1e-3)
    n = 2
    ws_ = (ctypes.c_void_p * n)(FAKE, FAKE)
    cs = (ctypes.c_void_p * n)(FAKE, FAKE)
    ps = (ctypes.c_void_p * n)(FAKE, FAKE)
    lds = (ctypes.c_int64 * n)(256, 512)
    ds = (ctypes.c_int64 * n)(64, 128)
    ks = (ctypes.c_int64 * n)(256, 512)
    seeds = (ctypes.c_uint64 * n)(1, 2)
    need = lib.rgc_apply_batch_workspace_size(n, ds, ks, 64)
    assert need > 0
    assert lib.rgc_apply_batch(0, None, None, None, None, None, None, 64, f, None, None, None, 0, s) == OK
    assert lib.rgc_apply_batch(17, ws_, lds, cs, ps, ds, ks, 64, f, seeds, None, FAKE, need, s) == UNSUP
    assert lib.rgc_apply_batch(n, ws_, lds, cs, ps, ds, ks, 64, f, None, None, FAKE, need, s) == NULL  # seeds
    bad_ld = (ctypes.c_int64 * n)(256, 500)
    assert lib.rgc_apply_batch(n, ws_, bad_ld, cs, ps, ds, ks, 64, f, seeds, None, FAKE, need, s) == SHAPE
    assert lib.rgc_apply_batch(n, ws_, lds, cs, ps, ds, ks, 72, f, seeds, None, FAKE, need, s) == UNSUP
    bad_c = (ctypes.c_void_p * n)(FAKE, FAKE + 4)
    assert lib.rgc_apply_batch(n, ws_, lds, bad_c, ps, ds, ks, 64, f, seeds, None, FAKE, need, s) == ALIGN
    assert lib.rgc_apply_batch(n, ws_, lds, cs, ps, ds, ks, 64, f, seeds, None, FAKE, need - 8, s) == WS
    # a matrix's workspace share does not depend on the rest of the batch
    one = lib.rgc_apply_workspace_size(64, 256, 64)
    assert 0 < one <= need


def test_scaled_apply_validation(lib):
    s = None
    f = ctypes.c_float(1e-3)
    assert lib.rgc_apply_scaled(FAKE, 255, FAKE, FAKE, 64, 256, 16, f, 0, s) == SHAPE
    assert lib.rgc_apply_scaled(FAKE, 256, FAKE, FAKE, 64, 256, 272, f, 0, s) == SHAPE  # r > k
    assert lib.rgc_apply_scaled(FAKE, 256, FAKE, FAKE, 60, 256, 16, f, 0, s) == UNSUP
    assert lib.rgc_apply_scaled(FAKE, 256, FAKE, None, 64, 256, 16, f, 0, s) == NULL
    assert lib.rgc_apply_scaled(FAKE + 8, 256, FAKE, FAKE, 64, 256, 16, f, 0, s) == ALIGN
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert lib.rgc_apply_scaled(FAKE, 256, FAKE, FAKE, 64, 256, 16, ctypes.c_float(bad), 0, s) == VALUE
    n = 2
    ws_ = (ctypes.c_void_p * n)(FAKE, FAKE)
    lds = (ctypes.c_int64 * n)(256, 512)
    ds = (ctypes.c_int64 * n)(64, 128)
    ks = (ctypes.c_int64 * n)(256, 512)
    seeds = (ctypes.c_uint64 * n)(1, 2)
    alphas = (ctypes.c_float * n)(1e-3, float("nan"))
    assert lib.rgc_apply_scaled_batch(0, None, None, None, None, None, None, 64, None, None, s) == OK
    assert lib.rgc_apply_scaled_batch(n, ws_, lds, ws_, ws_, ds, ks, 64, None, seeds, s) == NULL
    assert lib.rgc_apply_scaled_batch(n, ws_, lds, ws_, ws_, ds, ks, 64, alphas, seeds, s) == VALUE
    assert lib.rgc_apply_scaled_batch(17, ws_, lds, ws_, ws_, ds, ks, 64, alphas, seeds, s) == UNSUP


def test_carried_apply_validation(lib):
    s = None
    f = ctypes.c_float(1e-3)
    need = lib.rgc_apply_workspace_size(64, 256, 16)
    # the workspace holds one fp64 partial per update workgroup for the carried norm
    assert need >= 8 * 2
    args = lambda W=FAKE, ldw=256, C=FAKE, d=64, r=16, wn=FAKE, fresh=0, ws=FAKE, n=need: (
        W, ldw, C, FAKE, d, 256, r, f, 7, None, wn, fresh, ws, n, s)
    assert lib.rgc_apply_carried(*args(ldw=255)) == SHAPE
    assert lib.rgc_apply_carried(*args(r=272)) == SHAPE  # r > k
    assert lib.rgc_apply_carried(*args(d=60)) == UNSUP
    assert lib.rgc_apply_carried(*args(wn=None)) == NULL
    assert lib.rgc_apply_carried(*args(C=None, fresh=1)) == NULL
    assert lib.rgc_apply_carried(*args(wn=FAKE + 4)) == ALIGN
    assert lib.rgc_apply_carried(*args(ws=None)) == WS
    assert lib.rgc_apply_carried(*args(n=need - 8)) == WS
    assert lib.rgc_apply_carried(*args(ws=FAKE + 128)) == ALIGN
    n = 2
    ws_ = (ctypes.c_void_p * n)(FAKE, FAKE)
    lds = (ctypes.c_int64 * n)(256, 512)
    ds = (ctypes.c_int64 * n)(64, 128)
    ks = (ctypes.c_int64 * n)(256, 512)
    seeds = (ctypes.c_uint64 * n)(1, 2)
    assert lib.rgc_apply_carried_batch(0, None, None, None, None, None, None, 64, f, None, None, None, 0, None, 0,
                                       s) == OK
    assert lib.rgc_apply_carried_batch(n, ws_, lds, ws_, ws_, ds, ks, 64, f, seeds, None, None, 1, FAKE, 1 << 30,
                                       s) == NULL
    assert lib.rgc_apply_carried_batch(17, ws_, lds, ws_, ws_, ds, ks, 64, f, seeds, None, FAKE, 0, FAKE, 1 << 30,
                                       s) == UNSUP


def test_apply_from_seed_validation(lib):
    s = None
    f = ctypes.c_float(1e-3)
    need = lib.rgc_apply_from_seed_workspace_size(1, 2048, 1024, 64)
    # the regenerated P (bf16) plus the larger of the sampling and update scratch
    assert need >= 1024 * 64 * 2 + lib.rgc_sample_projection_workspace_size(1, 1024, 64)
    assert need >= 1024 * 64 * 2 + lib.rgc_apply_workspace_size(2048, 1024, 64)
    assert lib.rgc_apply_from_seed_workspace_size(1, 2048, 1024, 256) == 0  # QR limited to r <= 128
    assert lib.rgc_apply_from_seed_workspace_size(0, 2048, 1024, 256) > 1024 * 256 * 2
    args = lambda mode=0, kind=1, W=FAKE, ldw=1024, C=FAKE, d=2048, r=64, step=f, stats=None, ws=FAKE, n=need: (
        mode, kind, 5, W, ldw, C, d, 1024, r, step, 7, stats, ws, n, s)
    assert lib.rgc_apply_from_seed(*args(mode=2)) == UNSUP
    assert lib.rgc_apply_from_seed(*args(mode=1, stats=FAKE)) == UNSUP  # stats only with the normalized update
    assert lib.rgc_apply_from_seed(*args(ldw=1000)) == SHAPE
    assert lib.rgc_apply_from_seed(*args(r=2048)) == SHAPE  # r > k
    assert lib.rgc_apply_from_seed(*args(ws=None)) == WS
    assert lib.rgc_apply_from_seed(*args(n=need - 256)) == WS
    assert lib.rgc_apply_from_seed(*args(ws=FAKE + 128)) == ALIGN
    assert lib.rgc_apply_from_seed(*args(kind=1, r=256, n=1 << 30)) == UNSUP  # QR at r = 256
    assert lib.rgc_apply_from_seed(*args(C=None)) == NULL
    assert lib.rgc_apply_from_seed(*args(d=2044)) == UNSUP
    assert lib.rgc_apply_from_seed(*args(mode=1, step=ctypes.c_float(float("nan")))) == VALUE


def test_projection_validation(lib):
    s = None
    assert lib.rgc_sample_projection(0, 1, 64, 128, FAKE, None, 0, s) == SHAPE  # r > k
    assert lib.rgc_sample_projection(0, 1, 64, 24, FAKE, None, 0, s) == UNSUP
    assert lib.rgc_sample_projection(1, 1, 1024, 256, FAKE, None, 0, s) == UNSUP  # QR r > 128
    assert lib.rgc_sample_projection(7, 1, 1024, 64, FAKE, None, 0, s) == UNSUP
    assert lib.rgc_sample_projection(0, 1, 1024, 64, None, None, 0, s) == NULL
    assert lib.rgc_sample_projection(1, 1, 1024, 64, FAKE, None, 0, s) == WS
    assert lib.rgc_sample_projection(0, 1, 1024, 64, FAKE + 8, None, 0, s) == ALIGN


def test_batched_projection_validation(lib):
    s = None
    ks = (ctypes.c_int64 * 2)(1024, 2048)
    seeds = (ctypes.c_uint64 * 2)(1, 2)
    ps = (ctypes.c_void_p * 2)(FAKE, FAKE + 8)
    assert lib.rgc_sample_projections(1, 17, seeds, ks, 64, ps, None, 0, s) == UNSUP  # n > 16
    assert lib.rgc_sample_projections(1, 0, None, None, 64, None, None, 0, s) == OK
    assert lib.rgc_sample_projections(1, 2, None, ks, 64, ps, None, 0, s) == NULL
    assert lib.rgc_sample_projections(1, 2, seeds, ks, 64, ps, None, 0, s) == ALIGN  # second P misaligned
    ps[1] = FAKE
    assert lib.rgc_sample_projections(1, 2, seeds, ks, 64, ps, None, 0, s) == WS
    need = lib.rgc_sample_projections_workspace_size(1, 2, ks, 64)
    assert need == lib.rgc_sample_projection_workspace_size(1, 1024, 64) + lib.rgc_sample_projection_workspace_size(1, 2048, 64)


def test_test_hooks_validation(lib):
    s = None
    assert lib.rgc_test_philox(0, -1, FAKE, FAKE, s) == SHAPE
    assert lib.rgc_test_philox(0, 0, None, None, s) == OK
    assert lib.rgc_test_stochastic_round(FAKE, FAKE, 4, 8, 7, 0, 0, 0, s) == SHAPE
    assert lib.rgc_test_round_nearest(FAKE, FAKE, -1, s) == SHAPE
    assert lib.rgc_test_round_nearest(FAKE, FAKE, (1 << 31) + 1, s) == SHAPE
    assert lib.rgc_test_round_nearest(None, None, 0, s) == OK
    assert lib.rgc_test_round_nearest(None, FAKE, 4, s) == NULL
    assert lib.rgc_test_round_nearest(FAKE + 2, FAKE, 4, s) == ALIGN
    assert lib.rgc_test_reconstruct(FAKE, FAKE, FAKE, 64, 256, 24, s) == UNSUP


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(16, 64, dtype=torch.bfloat16)
    p = torch.zeros(64, 16, dtype=torch.bfloat16)
    with pytest.raises(rgc.RgcError):
        rgc.rgc_project(x, p)


def test_noalloc_rejects_oversized_calls_before_any_launch(lib):
    """rgc_apply_noalloc: a call whose workspace exceeds the static scratch
    returns RGC_ERR_SCRATCH on the host (no HIP call is made before it)."""
    SCRATCH = 8
    assert lib.rgc_apply_workspace_size(65536, 65536, 128) > (8 << 20)
    assert lib.rgc_apply_noalloc(FAKE, 65536, FAKE, FAKE, 65536, 65536, 128, 1e-3, 1, None, None) == SCRATCH
    assert b"scratch" in lib.rgc_status_string(SCRATCH)
    # the ordinary argument errors come first, as in rgc_apply
    assert lib.rgc_apply_noalloc(FAKE, 63, FAKE, FAKE, 16, 64, 16, 1e-3, 1, None, None) == SHAPE
    assert lib.rgc_apply_noalloc(None, 64, FAKE, FAKE, 16, 64, 16, 1e-3, 1, None, None) == NULL
    assert lib.rgc_apply_noalloc(FAKE, 64, FAKE, FAKE, 16, 64, 40, 1e-3, 1, None, None) == UNSUP


def test_small_ranks_are_supported(lib):
    """Ranks 4 and 8 are accepted by every workspace query (nonzero where a
    workspace is used); 12 is not a supported rank."""
    assert lib.rgc_sample_projection_workspace_size(1, 2048, 4) > 0  # QR at r = 4
    assert lib.rgc_sample_projection_workspace_size(1, 2048, 8) > 0
    assert lib.rgc_accumulate_workspace_size(4096, 2048, 4) > 0
    assert lib.rgc_apply_workspace_size(2048, 2048, 8) > 0
    assert lib.rgc_apply_workspace_size(2048, 2048, 12) == 0
    s = None
    assert lib.rgc_project(FAKE, 64, FAKE, FAKE, 16, 64, 12, None, 0, s) == UNSUP


def test_linear_validation(lib):
    """The layer products' host checks (nothing is launched: every call below
    is rejected, or has no tokens)."""
    s = None
    fwd = lib.rgc_linear_forward
    # X, ldx, W, ldw, P, Y, ldy, XP, T, d, k, r, stream
    assert fwd(None, 64, None, 64, None, None, 64, None, 0, 64, 64, 16, s) == OK  # no tokens
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, -1, 64, 64, 16, s) == SHAPE
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 16, 32, s) == SHAPE  # r > k
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 64, 24, s) == UNSUP  # rank
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 60, 16, s) == UNSUP  # k % 8
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 60, 64, 16, s) == UNSUP  # d % 8
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 1 << 17, 64, 64, 16, s) == UNSUP  # T above the limit
    assert fwd(FAKE, 64, FAKE, 64, None, FAKE, 64, FAKE, 16, 64, 64, 16, s) == NULL  # P
    assert fwd(FAKE, 64, None, 64, FAKE, FAKE, 64, FAKE, 16, 64, 64, 16, s) == NULL  # W
    assert fwd(FAKE + 2, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 64, 16, s) == ALIGN
    assert fwd(FAKE, 68, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 64, 16, s) == ALIGN  # ldx % 8
    assert fwd(FAKE, 64, FAKE, 64, FAKE, FAKE, 60, FAKE, 16, 64, 64, 16, s) == SHAPE  # ldy < d
    assert fwd(FAKE, (1 << 23) + 8, FAKE, 64, FAKE, FAKE, 64, FAKE, 16, 64, 64, 16, s) == UNSUP  # ldx > 2^23
    bwd = lib.rgc_linear_backward
    # D, ldd, W, ldw, XP, C, dX, lddx, T, d, k, r, ws, ws_bytes, stream
    assert bwd(FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, 64, 16, 64, 64, 24, None, 0, s) == UNSUP
    assert bwd(FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, 64, 16, 60, 64, 16, None, 0, s) == UNSUP  # d % 8
    assert bwd(FAKE, 64, FAKE, 60, FAKE, FAKE, FAKE, 64, 16, 64, 60, 16, None, 0, s) == UNSUP  # k % 8
    assert bwd(FAKE, 64, FAKE, 64, None, FAKE, FAKE, 64, 16, 64, 64, 16, None, 0, s) == NULL  # XP
    assert bwd(FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, 60, 16, 64, 64, 16, None, 0, s) == SHAPE  # lddx < k
    need = lib.rgc_linear_backward_workspace_size(4096, 2048, 2048, 64)
    assert need == lib.rgc_accumulate_workspace_size(4096, 2048, 64) and need > 0
    assert lib.rgc_linear_backward_workspace_size(4096, 2048, 2048, 0) == 0
    assert bwd(FAKE, 2048, FAKE, 2048, FAKE, FAKE, FAKE, 2048, 4096, 2048, 2048, 64, FAKE, need - 8, s) == WS
    assert bwd(FAKE, 2048, FAKE, 2048, FAKE, FAKE, FAKE, 2048, 4096, 2048, 2048, 64, FAKE + 16, need, s) == ALIGN


def test_apply_rejects_widths_not_divisible_by_8(lib):
    s = None
    f = ctypes.c_float(1e-3)
    assert lib.rgc_apply(FAKE, 260, FAKE, FAKE, 64, 260, 16, f, 0, None, FAKE, 1 << 20, s) == UNSUP  # k % 8
    assert lib.rgc_apply(FAKE, 256, FAKE, FAKE, 68, 256, 16, f, 0, None, FAKE, 1 << 20, s) == UNSUP  # d % 8


def test_deferred_accumulate_validation(lib):
    s = None
    n = 1
    dptr = (ctypes.c_void_p * n)(FAKE)
    lds = (ctypes.c_int64 * n)(256)
    ds = (ctypes.c_int64 * n)(256)
    fn = lib.rgc_accumulate_batch_deferred
    assert fn(n, dptr, lds, ds, dptr, dptr, 16, 64, None, 0, 4, s) == SHAPE  # phase out of range
    assert fn(n, dptr, lds, ds, dptr, dptr, 16, 64, None, 0, -1, s) == SHAPE
    assert fn(0, None, None, None, None, None, 16, 64, None, 0, 1, s) == OK
    assert fn(n, dptr, lds, ds, dptr, dptr, 16, 72, None, 0, 1, s) == UNSUP  # rank

