"""Thin Python binding of librgc (the gfx950 sketch library), through ctypes.

Argument marshalling only: every step runs in the HIP kernels of librgc.so.
torch supplies device memory and the current HIP stream. There is no CPU
fallback: if the library is missing or a GPU is absent, calls raise.

Names mirror the C ABI in include/rgc.h:
  rgc_sample_projection(kind, seed, k, r)  -> P (k x r bf16)
  rgc_project(X, P)                         -> XP = bf16(X P)
  rgc_accumulate(D, XP, C)                  C += D^T XP (in place)
  rgc_apply(W, C, P, tau, seed)             W <- SR(W - tau ||W|| H / ||H||) (in place)
  rgc_apply_scaled(W, C, P, alpha, seed)    W <- SR(W - alpha H) (in place)
  rgc_apply_carried(W, C, P, tau, seed, wnorm2, fresh)
                                            rgc_apply with ||W||^2 carried between calls
  rgc_apply_from_seed(mode, kind, proj_seed, W, C, step, seed)
                                            P regenerated from its seed, then one of the two
  rgc_linear_forward(X, W, P)               (Y, XP) = (bf16(X W^T), bf16(X P)), one tile grid
  rgc_linear_backward(D, W, XP, C)          dX = bf16(D W), then C += D^T XP
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "librgc.so")

RGC_PROJ_RADEMACHER = 0
RGC_PROJ_QR_GAUSSIAN = 1
_KINDS = {"rademacher": RGC_PROJ_RADEMACHER, "qr": RGC_PROJ_QR_GAUSSIAN}
RGC_UPDATE_NORMALIZED = 0
RGC_UPDATE_SCALED = 1
_MODES = {"normalized": RGC_UPDATE_NORMALIZED, "scaled": RGC_UPDATE_SCALED}

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_f32 = ctypes.c_float

# (name, restype, argtypes) for every exported function of include/rgc.h
SIGNATURES = {
    "rgc_abi_version": (ctypes.c_int, []),
    "rgc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rgc_sample_projection_workspace_size": (_sz, [ctypes.c_int, _i64, _i64]),
    "rgc_sample_projection": (ctypes.c_int, [ctypes.c_int, _u64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "rgc_sample_projections_workspace_size": (_sz, [ctypes.c_int, _i64, ctypes.POINTER(_i64), _i64]),
    "rgc_sample_projections": (ctypes.c_int, [ctypes.c_int, _i64, ctypes.POINTER(_u64), ctypes.POINTER(_i64), _i64,
                                               ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "rgc_project_workspace_size": (_sz, [_i64, _i64, _i64]),
    "rgc_project": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "rgc_project_batch_workspace_size": (_sz, [_i64, ctypes.POINTER(_i64), _i64, _i64]),
    "rgc_project_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                         ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64, _i64, _vp, _sz, _vp]),
    "rgc_accumulate_workspace_size": (_sz, [_i64, _i64, _i64]),
    "rgc_accumulate_batch_workspace_size": (_sz, [_i64, ctypes.POINTER(_i64), _i64, _i64]),
    "rgc_accumulate_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                            ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64, _i64, _vp, _sz, _vp]),
    "rgc_accumulate": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "rgc_accumulate_batch_deferred": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                                     ctypes.POINTER(_i64), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                     _i64, _i64, _vp, _sz, ctypes.c_int, _vp]),
    "rgc_test_accumulate_batch_deferred_wgs": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                                              ctypes.POINTER(_i64), ctypes.POINTER(_vp),
                                                              ctypes.POINTER(_vp), _i64, _i64, _vp, _sz, ctypes.c_int,
                                                              _vp]),
    "rgc_apply_workspace_size": (_sz, [_i64, _i64, _i64]),
    "rgc_apply_batch_workspace_size": (_sz, [_i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64]),
    "rgc_apply_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_vp),
                                       ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64, _f32,
                                       ctypes.POINTER(_u64), ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "rgc_apply": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _f32, _u64, _vp, _vp, _sz, _vp]),
    "rgc_apply_scaled": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _f32, _u64, _vp]),
    "rgc_apply_noalloc": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _f32, _u64, _vp, _vp]),
    "rgc_apply_scaled_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_vp),
                                              ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64,
                                              ctypes.POINTER(_f32), ctypes.POINTER(_u64), _vp]),
    "rgc_apply_carried_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_vp),
                                               ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64,
                                               _f32, ctypes.POINTER(_u64), ctypes.POINTER(_vp), _vp, ctypes.c_int,
                                               _vp, _sz, _vp]),
    "rgc_apply_carried": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _f32, _u64, _vp, _vp, ctypes.c_int,
                                         _vp, _sz, _vp]),
    "rgc_apply_from_seed_workspace_size": (_sz, [ctypes.c_int, _i64, _i64, _i64]),
    "rgc_apply_from_seed": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _u64, _vp, _i64, _vp, _i64, _i64, _i64, _f32,
                                           _u64, _vp, _vp, _sz, _vp]),
    "rgc_linear_forward": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]),
    "rgc_linear_forward_batch": (ctypes.c_int, [_i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                                ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                                ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                                ctypes.POINTER(_vp), _i64, _i64, _vp]),
    "rgc_linear_backward_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "rgc_linear_backward": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _sz,
                                           _vp]),
    "rgc_test_philox": (ctypes.c_int, [_u64, _i64, _vp, _vp, _vp]),
    "rgc_test_stochastic_round": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _u64, _vp]),
    "rgc_test_round_nearest": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "rgc_test_reconstruct": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "rgc_test_sketch_workspace_size": (_sz, [ctypes.c_int, _i64, _i64, ctypes.POINTER(_i64), _i64, _i64]),
    "rgc_project_shared_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "rgc_project_shared": (ctypes.c_int, [_i64, _vp, _i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64, _i64,
                                          _vp, _sz, _vp]),
    "rgc_test_project_shared_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "rgc_test_project_shared_wgs": (ctypes.c_int, [_i64, _i64, _vp, _i64, _i64, ctypes.POINTER(_vp),
                                                   ctypes.POINTER(_vp), _i64, _i64, _vp, _sz, _vp]),
    "rgc_test_project_batch_wgs": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                                  ctypes.POINTER(_i64), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                  _i64, _i64, _vp, _sz, _vp]),
    "rgc_test_accumulate_batch_wgs": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                                     ctypes.POINTER(_i64), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                     _i64, _i64, _vp, _sz, _vp]),
}

_lib = None
_lib_lock = threading.Lock()


class RgcError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads librgc.so and declares its signatures (no GPU needed)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RgcError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def abi_version() -> int:
    return load_library().rgc_abi_version()


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().rgc_status_string(status).decode()
        raise RgcError(f"librgc status {status}: {msg}")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu(*tensors: torch.Tensor) -> torch.device:
    dev = tensors[0].device
    if dev.type != "cuda":
        raise RgcError("librgc runs on the GPU only: tensors must be on a cuda (HIP) device")
    for t in tensors:
        if t.device != dev:
            raise RgcError("all tensors must be on the same device")
    return dev


def _rows(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    """Checks a row-major 2-D tensor (unit column stride) and returns its row stride."""
    if t.dtype != dtype:
        raise RgcError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise RgcError(f"{name} must be 2-D with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _dense(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype or not t.is_contiguous():
        raise RgcError(f"{name} must be a contiguous {dtype} tensor")


class Workspace:
    """Device scratch for the calls ordered on one stream, grown on demand.

    Workspace contents are dead after each call's kernels complete, so one
    buffer serves every call ordered on a stream. The exception is a deferred
    accumulation (rgc_accumulate_batch_deferred), whose partial sums live in
    its workspace from the first call to the last: give it a Workspace of its
    own.
    """

    def __init__(self, device: torch.device):
        self.device = device
        self.buf = torch.zeros(0, dtype=torch.uint8, device=device)

    def get(self, nbytes: int) -> tuple[ctypes.c_void_p, int]:
        if nbytes == 0:
            return ctypes.c_void_p(self.buf.data_ptr() if self.buf.numel() else 0), self.buf.numel()
        if self.buf.numel() < nbytes:
            self.buf = torch.empty(((nbytes + 4095) // 4096) * 4096, dtype=torch.uint8, device=self.device)
        return ctypes.c_void_p(self.buf.data_ptr()), self.buf.numel()


_workspaces: dict = {}


def default_workspace(dev: torch.device) -> Workspace:
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = Workspace(torch.device("cuda", key[0]))
        _workspaces[key] = ws
    return ws


def rgc_sample_projection(kind: str, seed: int, k: int, r: int, out: torch.Tensor | None = None,
                          device=None, workspace: Workspace | None = None) -> torch.Tensor:
    lib = load_library()
    if out is None:
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        out = torch.empty((k, r), dtype=torch.bfloat16, device=dev)
    dev = _need_gpu(out)
    _dense(out, torch.bfloat16, "P")
    kid = _KINDS[kind]
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_sample_projection_workspace_size(kid, k, r))
    _check(lib.rgc_sample_projection(kid, seed & 0xFFFFFFFFFFFFFFFF, k, r, out.data_ptr(), wp, wn, _stream(dev)))
    return out


def rgc_sample_projections(kind: str, seeds, Ps, workspace: Workspace | None = None):
    """Fills each P in Ps (k_m x r bf16) as rgc_sample_projection(kind, seeds[m], ...), in one batch."""
    lib = load_library()
    n = len(Ps)
    if n == 0:
        return Ps
    dev = _need_gpu(*Ps)
    r = Ps[0].shape[1]
    for p in Ps:
        _dense(p, torch.bfloat16, "P")
        if p.shape[1] != r:
            raise RgcError("all projections in a batch share one rank")
    kid = _KINDS[kind]
    ks = (_i64 * n)(*[p.shape[0] for p in Ps])
    sd = (_u64 * n)(*[s & 0xFFFFFFFFFFFFFFFF for s in seeds])
    ptrs = (_vp * n)(*[p.data_ptr() for p in Ps])
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_sample_projections_workspace_size(kid, n, ks, r))
    _check(lib.rgc_sample_projections(kid, n, sd, ks, r, ptrs, wp, wn, _stream(dev)))
    return Ps


def rgc_project(X: torch.Tensor, P: torch.Tensor, out: torch.Tensor | None = None,
                workspace: Workspace | None = None) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(X, P)
    ldx = _rows(X, torch.bfloat16, "X")
    _dense(P, torch.bfloat16, "P")
    T, k = X.shape
    r = P.shape[1]
    if P.shape[0] != k:
        raise RgcError("P must be k x r with k = X.shape[1]")
    if out is None:
        out = torch.empty((T, r), dtype=torch.bfloat16, device=dev)
    _dense(out, torch.bfloat16, "XP")
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_project_workspace_size(T, k, r))
    _check(lib.rgc_project(X.data_ptr(), ldx, P.data_ptr(), out.data_ptr(), T, k, r, wp, wn, _stream(dev)))
    return out


def rgc_accumulate(D: torch.Tensor, XP: torch.Tensor, C: torch.Tensor, workspace: Workspace | None = None) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(D, XP, C)
    ldd = _rows(D, torch.bfloat16, "D")
    _dense(XP, torch.bfloat16, "XP")
    _dense(C, torch.float32, "C")
    T, d = D.shape
    r = XP.shape[1]
    if XP.shape[0] != T or tuple(C.shape) != (d, r):
        raise RgcError("shapes must be D: T x d, XP: T x r, C: d x r")
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_accumulate_workspace_size(T, d, r))
    _check(lib.rgc_accumulate(D.data_ptr(), ldd, XP.data_ptr(), C.data_ptr(), T, d, r, wp, wn, _stream(dev)))
    return C


def _ptrs(ts):
    return (_vp * len(ts))(*[t.data_ptr() for t in ts])


def _i64s(vals):
    return (_i64 * len(vals))(*vals)


def rgc_project_batch(Xs, Ps, outs=None, workspace: Workspace | None = None):
    """XPs[m] = bf16(Xs[m] Ps[m]) for all m in one launch (one rank, one token count)."""
    lib = load_library()
    n = len(Xs)
    if n == 0:
        return []
    dev = _need_gpu(*Xs, *Ps)
    T = Xs[0].shape[0]
    r = Ps[0].shape[1]
    ldxs, ks = [], []
    for x, p in zip(Xs, Ps):
        ldxs.append(_rows(x, torch.bfloat16, "X"))
        _dense(p, torch.bfloat16, "P")
        if x.shape[0] != T or p.shape[1] != r or p.shape[0] != x.shape[1]:
            raise RgcError("batch items must share T and r, with P of shape (X.shape[1], r)")
        ks.append(x.shape[1])
    if outs is None:
        outs = [torch.empty((T, r), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    for o in outs:
        _dense(o, torch.bfloat16, "XP")
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_project_batch_workspace_size(n, _i64s(ks), T, r))
    _check(lib.rgc_project_batch(n, _ptrs(Xs), _i64s(ldxs), _i64s(ks), _ptrs(Ps), _ptrs(outs), T, r, wp, wn,
                                 _stream(dev)))
    return outs


def rgc_project_shared(X: torch.Tensor, Ps, outs=None, workspace: Workspace | None = None, workgroups: int = 0):
    """XPs[i] = bf16(X Ps[i]) for the projections of matrices that read the same
    X, with X streamed once for all of them (n <= 4, n * r <= 256).
    workgroups > 0 forces the workgroup count (test hook)."""
    lib = load_library()
    n = len(Ps)
    if n == 0:
        return []
    dev = _need_gpu(X, *Ps)
    ldx = _rows(X, torch.bfloat16, "X")
    T, k = X.shape
    r = Ps[0].shape[1]
    for p in Ps:
        _dense(p, torch.bfloat16, "P")
        if tuple(p.shape) != (k, r):
            raise RgcError("every P must be k x r with k = X.shape[1] and one rank r")
    if outs is None:
        outs = [torch.empty((T, r), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    for o in outs:
        _dense(o, torch.bfloat16, "XP")
    if workgroups > 0:
        nbytes = lib.rgc_test_project_shared_workspace_size(workgroups, n, T, k, r)
        buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        _check(lib.rgc_test_project_shared_wgs(workgroups, n, X.data_ptr(), ldx, k, _ptrs(Ps), _ptrs(outs), T, r,
                                               buf.data_ptr(), buf.numel(), _stream(dev)))
        return outs
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_project_shared_workspace_size(n, T, k, r))
    _check(lib.rgc_project_shared(n, X.data_ptr(), ldx, k, _ptrs(Ps), _ptrs(outs), T, r, wp, wn, _stream(dev)))
    return outs


def rgc_accumulate_batch(Ds, XPs, Cs, workspace: Workspace | None = None):
    """Cs[m] += Ds[m]^T XPs[m] for all m in one launch (one rank, one token count)."""
    lib = load_library()
    n = len(Ds)
    if n == 0:
        return Cs
    dev = _need_gpu(*Ds, *XPs, *Cs)
    T = Ds[0].shape[0]
    r = XPs[0].shape[1]
    ldds, ds = [], []
    for dd, xp, c in zip(Ds, XPs, Cs):
        ldds.append(_rows(dd, torch.bfloat16, "D"))
        _dense(xp, torch.bfloat16, "XP")
        _dense(c, torch.float32, "C")
        if dd.shape[0] != T or tuple(xp.shape) != (T, r) or tuple(c.shape) != (dd.shape[1], r):
            raise RgcError("batch items must share T and r: D T x d, XP T x r, C d x r")
        ds.append(dd.shape[1])
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_accumulate_batch_workspace_size(n, _i64s(ds), T, r))
    _check(lib.rgc_accumulate_batch(n, _ptrs(Ds), _i64s(ldds), _i64s(ds), _ptrs(XPs), _ptrs(Cs), T, r, wp, wn,
                                    _stream(dev)))
    return Cs


def rgc_accumulate_batch_deferred(Ds, XPs, Cs, workspace: Workspace, first: bool, last: bool,
                                  workgroups: int = 0):
    """Cs[m] += Ds[m]^T XPs[m] as one call of an accumulation over several
    microbatches whose split-tile partial sums stay in `workspace` between the
    calls and reach C in the call with last=True. The workspace is required:
    it carries state from the first call to the last, so no other call may
    use it in between. workgroups > 0 forces the workgroup count (test hook;
    the same count for every call of the accumulation)."""
    lib = load_library()
    n = len(Ds)
    if n == 0:
        return Cs
    if workspace is None:
        raise RgcError("a deferred accumulation needs its own workspace")
    dev = _need_gpu(*Ds, *XPs, *Cs)
    T = Ds[0].shape[0]
    r = XPs[0].shape[1]
    ldds, ds = [], []
    for dd, xp, c in zip(Ds, XPs, Cs):
        ldds.append(_rows(dd, torch.bfloat16, "D"))
        _dense(xp, torch.bfloat16, "XP")
        _dense(c, torch.float32, "C")
        if dd.shape[0] != T or tuple(xp.shape) != (T, r) or tuple(c.shape) != (dd.shape[1], r):
            raise RgcError("batch items must share T and r: D T x d, XP T x r, C d x r")
        ds.append(dd.shape[1])
    phase = (1 if first else 0) | (2 if last else 0)
    if workgroups > 0:
        wp, wn = workspace.get(lib.rgc_test_sketch_workspace_size(1, workgroups, n, _i64s(ds), T, r))
        _check(lib.rgc_test_accumulate_batch_deferred_wgs(workgroups, n, _ptrs(Ds), _i64s(ldds), _i64s(ds),
                                                          _ptrs(XPs), _ptrs(Cs), T, r, wp, wn, phase, _stream(dev)))
        return Cs
    wp, wn = workspace.get(lib.rgc_accumulate_batch_workspace_size(n, _i64s(ds), T, r))
    _check(lib.rgc_accumulate_batch_deferred(n, _ptrs(Ds), _i64s(ldds), _i64s(ds), _ptrs(XPs), _ptrs(Cs), T, r, wp,
                                             wn, phase, _stream(dev)))
    return Cs


def rgc_apply(W: torch.Tensor, C: torch.Tensor, P: torch.Tensor, tau: float, seed: int,
              stats: torch.Tensor | None = None, workspace: Workspace | None = None) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(W, C, P)
    ldw = _rows(W, torch.bfloat16, "W")
    _dense(C, torch.float32, "C")
    _dense(P, torch.bfloat16, "P")
    d, k = W.shape
    r = C.shape[1]
    if tuple(C.shape) != (d, r) or tuple(P.shape) != (k, r):
        raise RgcError("shapes must be W: d x k, C: d x r, P: k x r")
    sp = None
    if stats is not None:
        _need_gpu(stats)
        _dense(stats, torch.float32, "stats")
        if stats.numel() < 4:
            raise RgcError("stats needs 4 floats")
        sp = stats.data_ptr()
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_apply_workspace_size(d, k, r))
    _check(lib.rgc_apply(W.data_ptr(), ldw, C.data_ptr(), P.data_ptr(), d, k, r, float(tau),
                         seed & 0xFFFFFFFFFFFFFFFF, sp, wp, wn, _stream(dev)))
    return W


def rgc_apply_noalloc(W: torch.Tensor, C: torch.Tensor, P: torch.Tensor, tau: float, seed: int,
                      stats: torch.Tensor | None = None) -> torch.Tensor:
    """rgc_apply without a workspace: the library's static device scratch is
    used instead (no device allocation on any path of this call)."""
    lib = load_library()
    dev = _need_gpu(W, C, P)
    ldw = _rows(W, torch.bfloat16, "W")
    _dense(C, torch.float32, "C")
    _dense(P, torch.bfloat16, "P")
    d, k = W.shape
    r = C.shape[1]
    if tuple(C.shape) != (d, r) or tuple(P.shape) != (k, r):
        raise RgcError("shapes must be W: d x k, C: d x r, P: k x r")
    sp = None
    if stats is not None:
        _need_gpu(stats)
        _dense(stats, torch.float32, "stats")
        if stats.numel() < 4:
            raise RgcError("stats needs 4 floats")
        sp = stats.data_ptr()
    _check(lib.rgc_apply_noalloc(W.data_ptr(), ldw, C.data_ptr(), P.data_ptr(), d, k, r, float(tau),
                                 seed & 0xFFFFFFFFFFFFFFFF, sp, _stream(dev)))
    return W


def rgc_apply_batch(Ws, Cs, Ps, tau: float, seeds, stats=None, workspace: Workspace | None = None):
    """rgc_apply for several matrices of one rank in three launches (one seed
    per matrix; stats: None or a list of device float[4] tensors or Nones)."""
    lib = load_library()
    n = len(Ws)
    if n == 0:
        return Ws
    if len(Cs) != n or len(Ps) != n or len(seeds) != n or (stats is not None and len(stats) != n):
        raise RgcError("Ws, Cs, Ps, seeds (and stats) must have the same length")
    dev = _need_gpu(*Ws, *Cs, *Ps)
    r = Cs[0].shape[1]
    ldws, ds, ks = [], [], []
    for W, C, P in zip(Ws, Cs, Ps):
        ldws.append(_rows(W, torch.bfloat16, "W"))
        _dense(C, torch.float32, "C")
        _dense(P, torch.bfloat16, "P")
        d, k = W.shape
        if tuple(C.shape) != (d, r) or tuple(P.shape) != (k, r):
            raise RgcError("batch items must share r: W d x k, C d x r, P k x r")
        ds.append(d)
        ks.append(k)
    sps = None
    if stats is not None:
        vals = []
        for st in stats:
            if st is None:
                vals.append(None)
                continue
            _need_gpu(st)
            _dense(st, torch.float32, "stats")
            if st.numel() < 4:
                raise RgcError("stats needs 4 floats")
            vals.append(st.data_ptr())
        sps = (_vp * n)(*vals)
    seeds_arr = (_u64 * n)(*[s & 0xFFFFFFFFFFFFFFFF for s in seeds])
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_apply_batch_workspace_size(n, _i64s(ds), _i64s(ks), r))
    _check(lib.rgc_apply_batch(n, _ptrs(Ws), _i64s(ldws), _ptrs(Cs), _ptrs(Ps), _i64s(ds), _i64s(ks), r,
                               float(tau), seeds_arr, sps, wp, wn, _stream(dev)))
    return Ws


def _stats_ptrs(stats, n):
    if stats is None:
        return None
    vals = []
    for st in stats:
        if st is None:
            vals.append(None)
            continue
        _need_gpu(st)
        _dense(st, torch.float32, "stats")
        if st.numel() < 4:
            raise RgcError("stats needs 4 floats")
        vals.append(st.data_ptr())
    return (_vp * n)(*vals)


def rgc_apply_carried_batch(Ws, Cs, Ps, tau: float, seeds, wnorm2: torch.Tensor, fresh: bool, stats=None,
                            workspace: Workspace | None = None):
    """rgc_apply_batch with ||W||^2 carried in wnorm2 (device float64, n values):
    fresh=True streams it from W first; on return wnorm2 holds ||W'||^2 of
    the weights written, for the next call with fresh=False."""
    lib = load_library()
    n = len(Ws)
    if n == 0:
        return Ws
    if len(Cs) != n or len(Ps) != n or len(seeds) != n or (stats is not None and len(stats) != n):
        raise RgcError("Ws, Cs, Ps, seeds (and stats) must have the same length")
    dev = _need_gpu(*Ws, *Cs, *Ps, wnorm2)
    _dense(wnorm2, torch.float64, "wnorm2")
    if wnorm2.numel() < n:
        raise RgcError("wnorm2 needs one float64 per matrix")
    r, ldws, ds, ks = _apply_items(Ws, Cs, Ps)
    sps = _stats_ptrs(stats, n)
    seeds_arr = (_u64 * n)(*[s & 0xFFFFFFFFFFFFFFFF for s in seeds])
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_apply_batch_workspace_size(n, _i64s(ds), _i64s(ks), r))
    _check(lib.rgc_apply_carried_batch(n, _ptrs(Ws), _i64s(ldws), _ptrs(Cs), _ptrs(Ps), _i64s(ds), _i64s(ks), r,
                                       float(tau), seeds_arr, sps, wnorm2.data_ptr(), 1 if fresh else 0, wp, wn,
                                       _stream(dev)))
    return Ws


def rgc_apply_carried(W: torch.Tensor, C: torch.Tensor, P: torch.Tensor, tau: float, seed: int,
                      wnorm2: torch.Tensor, fresh: bool, stats: torch.Tensor | None = None,
                      workspace: Workspace | None = None) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(W, C, P, wnorm2)
    _dense(wnorm2, torch.float64, "wnorm2")
    if wnorm2.numel() < 1:
        raise RgcError("wnorm2 needs one float64")
    r, ldws, ds, ks = _apply_items([W], [C], [P])
    sps = _stats_ptrs(None if stats is None else [stats], 1)
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_apply_workspace_size(ds[0], ks[0], r))
    _check(lib.rgc_apply_carried(W.data_ptr(), ldws[0], C.data_ptr(), P.data_ptr(), ds[0], ks[0], r, float(tau),
                                 seed & 0xFFFFFFFFFFFFFFFF, None if sps is None else sps[0], wnorm2.data_ptr(),
                                 1 if fresh else 0, wp, wn, _stream(dev)))
    return W


def _apply_items(Ws, Cs, Ps):
    r = Cs[0].shape[1]
    ldws, ds, ks = [], [], []
    for W, C, P in zip(Ws, Cs, Ps):
        ldws.append(_rows(W, torch.bfloat16, "W"))
        _dense(C, torch.float32, "C")
        _dense(P, torch.bfloat16, "P")
        d, k = W.shape
        if tuple(C.shape) != (d, r) or tuple(P.shape) != (k, r):
            raise RgcError("items must share r: W d x k, C d x r, P k x r")
        ds.append(d)
        ks.append(k)
    return r, ldws, ds, ks


def rgc_apply_scaled_batch(Ws, Cs, Ps, alphas, seeds):
    """W <- SR(W - alpha H) for several matrices of one rank in one launch."""
    lib = load_library()
    n = len(Ws)
    if n == 0:
        return Ws
    if len(Cs) != n or len(Ps) != n or len(alphas) != n or len(seeds) != n:
        raise RgcError("Ws, Cs, Ps, alphas and seeds must have the same length")
    dev = _need_gpu(*Ws, *Cs, *Ps)
    r, ldws, ds, ks = _apply_items(Ws, Cs, Ps)
    alphas_arr = (_f32 * n)(*[float(a) for a in alphas])
    seeds_arr = (_u64 * n)(*[s & 0xFFFFFFFFFFFFFFFF for s in seeds])
    _check(lib.rgc_apply_scaled_batch(n, _ptrs(Ws), _i64s(ldws), _ptrs(Cs), _ptrs(Ps), _i64s(ds), _i64s(ks), r,
                                      alphas_arr, seeds_arr, _stream(dev)))
    return Ws


def rgc_apply_scaled(W: torch.Tensor, C: torch.Tensor, P: torch.Tensor, alpha: float, seed: int) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(W, C, P)
    r, ldws, ds, ks = _apply_items([W], [C], [P])
    _check(lib.rgc_apply_scaled(W.data_ptr(), ldws[0], C.data_ptr(), P.data_ptr(), ds[0], ks[0], r, float(alpha),
                                seed & 0xFFFFFFFFFFFFFFFF, _stream(dev)))
    return W


def rgc_apply_from_seed(mode: str, kind: str, proj_seed: int, W: torch.Tensor, C: torch.Tensor, step: float,
                        seed: int, stats: torch.Tensor | None = None,
                        workspace: Workspace | None = None) -> torch.Tensor:
    """Regenerates P (kind, proj_seed) in the workspace and applies the update
    (mode "normalized": tau = step; "scaled": alpha = step)."""
    lib = load_library()
    dev = _need_gpu(W, C)
    ldw = _rows(W, torch.bfloat16, "W")
    _dense(C, torch.float32, "C")
    d, k = W.shape
    r = C.shape[1]
    if C.shape[0] != d:
        raise RgcError("shapes must be W: d x k, C: d x r")
    sp = None
    if stats is not None:
        _need_gpu(stats)
        _dense(stats, torch.float32, "stats")
        if stats.numel() < 4:
            raise RgcError("stats needs 4 floats")
        sp = stats.data_ptr()
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_apply_from_seed_workspace_size(_KINDS[kind], d, k, r))
    _check(lib.rgc_apply_from_seed(_MODES[mode], _KINDS[kind], proj_seed & 0xFFFFFFFFFFFFFFFF, W.data_ptr(), ldw,
                                   C.data_ptr(), d, k, r, float(step), seed & 0xFFFFFFFFFFFFFFFF, sp, wp, wn,
                                   _stream(dev)))
    return W


# ---- test hooks -------------------------------------------------------------

def rgc_test_philox(seed: int, ctr: torch.Tensor) -> torch.Tensor:
    """ctr: (n, 4) int32 tensor of counter words (bit patterns); returns (n, 4) int32."""
    lib = load_library()
    dev = _need_gpu(ctr)
    _dense(ctr, torch.int32, "ctr")
    out = torch.empty_like(ctr)
    _check(lib.rgc_test_philox(seed & 0xFFFFFFFFFFFFFFFF, ctr.shape[0], ctr.data_ptr(), out.data_ptr(), _stream(dev)))
    return out


def rgc_test_stochastic_round(v: torch.Tensor, seed: int, row0: int = 0, col0: int = 0) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(v)
    _dense(v, torch.float32, "v")
    rows, cols = v.shape
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _check(lib.rgc_test_stochastic_round(v.data_ptr(), out.data_ptr(), rows, cols, cols, row0, col0,
                                         seed & 0xFFFFFFFFFFFFFFFF, _stream(dev)))
    return out


def rgc_test_round_nearest(v: torch.Tensor) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(v)
    _dense(v, torch.float32, "v")
    out = torch.empty(v.shape, dtype=torch.bfloat16, device=dev)
    _check(lib.rgc_test_round_nearest(v.data_ptr(), out.data_ptr(), v.numel(), _stream(dev)))
    return out


def rgc_test_reconstruct(C: torch.Tensor, P: torch.Tensor) -> torch.Tensor:
    lib = load_library()
    dev = _need_gpu(C, P)
    _dense(C, torch.float32, "C")
    _dense(P, torch.bfloat16, "P")
    d, r = C.shape
    k = P.shape[0]
    H = torch.empty((d, k), dtype=torch.float32, device=dev)
    _check(lib.rgc_test_reconstruct(C.data_ptr(), P.data_ptr(), H.data_ptr(), d, k, r, _stream(dev)))
    return H


def rgc_test_project_batch_wgs(workgroups: int, Xs, Ps):
    """rgc_project_batch with a caller-given workgroup count (test hook)."""
    lib = load_library()
    n = len(Xs)
    dev = _need_gpu(*Xs, *Ps)
    T, r = Xs[0].shape[0], Ps[0].shape[1]
    ldxs = [_rows(x, torch.bfloat16, "X") for x in Xs]
    ks = [x.shape[1] for x in Xs]
    for p in Ps:
        _dense(p, torch.bfloat16, "P")
    outs = [torch.empty((T, r), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    nbytes = lib.rgc_test_sketch_workspace_size(0, workgroups, n, _i64s(ks), T, r)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.rgc_test_project_batch_wgs(workgroups, n, _ptrs(Xs), _i64s(ldxs), _i64s(ks), _ptrs(Ps), _ptrs(outs),
                                          T, r, ws.data_ptr(), ws.numel(), _stream(dev)))
    return outs


def rgc_test_accumulate_batch_wgs(workgroups: int, Ds, XPs, Cs):
    """rgc_accumulate_batch with a caller-given workgroup count (test hook)."""
    lib = load_library()
    n = len(Ds)
    dev = _need_gpu(*Ds, *XPs, *Cs)
    T, r = Ds[0].shape[0], XPs[0].shape[1]
    ldds = [_rows(d, torch.bfloat16, "D") for d in Ds]
    ds = [d.shape[1] for d in Ds]
    for x in XPs:
        _dense(x, torch.bfloat16, "XP")
    for c in Cs:
        _dense(c, torch.float32, "C")
    nbytes = lib.rgc_test_sketch_workspace_size(1, workgroups, n, _i64s(ds), T, r)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.rgc_test_accumulate_batch_wgs(workgroups, n, _ptrs(Ds), _i64s(ldds), _i64s(ds), _ptrs(XPs),
                                             _ptrs(Cs), T, r, ws.data_ptr(), ws.numel(), _stream(dev)))
    return Cs


def rgc_linear_forward(X: torch.Tensor, W: torch.Tensor, P: torch.Tensor | None = None,
                       Y: torch.Tensor | None = None, XP: torch.Tensor | None = None):
    """(Y, XP) = (bf16(X W^T), bf16(X P)) from one tile grid over [W^T | P]'s
    columns; XP is None when P is None. X: T x k (row stride >= k), W: d x k,
    P: k x r."""
    lib = load_library()
    dev = _need_gpu(X, W, *([P] if P is not None else []))
    ldx = _rows(X, torch.bfloat16, "X")
    ldw = _rows(W, torch.bfloat16, "W")
    T, k = X.shape
    d = W.shape[0]
    if W.shape[1] != k:
        raise RgcError("W must be d x k with k = X.shape[1]")
    r = 0
    if P is not None:
        _dense(P, torch.bfloat16, "P")
        if P.shape[0] != k:
            raise RgcError("P must be k x r with k = X.shape[1]")
        r = P.shape[1]
        if XP is None:
            XP = torch.empty((T, r), dtype=torch.bfloat16, device=dev)
        _dense(XP, torch.bfloat16, "XP")
    if Y is None:
        Y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    ldy = _rows(Y, torch.bfloat16, "Y")
    _check(lib.rgc_linear_forward(X.data_ptr(), ldx, W.data_ptr(), ldw, P.data_ptr() if P is not None else None,
                                  Y.data_ptr(), ldy, XP.data_ptr() if XP is not None else None, T, d, k, r,
                                  _stream(dev)))
    return Y, XP


def rgc_linear_forward_batch(Xs, Ws, Ps=None):
    """rgc_linear_forward for n <= 16 layers of one token count and one rank in
    one launch (items may share X). Returns (Ys, XPs)."""
    lib = load_library()
    n = len(Xs)
    if n == 0:
        return [], []
    dev = _need_gpu(*Xs, *Ws, *(Ps or []))
    T = Xs[0].shape[0]
    r = Ps[0].shape[1] if Ps else 0
    ldxs, ldws, ks, ds = [], [], [], []
    for m in range(n):
        ldxs.append(_rows(Xs[m], torch.bfloat16, "X"))
        ldws.append(_rows(Ws[m], torch.bfloat16, "W"))
        if Xs[m].shape[0] != T or Ws[m].shape[1] != Xs[m].shape[1]:
            raise RgcError("batch items must share T, with W of shape (d, X.shape[1])")
        if Ps:
            _dense(Ps[m], torch.bfloat16, "P")
            if tuple(Ps[m].shape) != (Xs[m].shape[1], r):
                raise RgcError("every P must be k x r with one rank r")
        ks.append(Xs[m].shape[1])
        ds.append(Ws[m].shape[0])
    Ys = [torch.empty((T, d), dtype=torch.bfloat16, device=dev) for d in ds]
    XPs = [torch.empty((T, r), dtype=torch.bfloat16, device=dev) for _ in range(n)] if Ps else None
    _check(lib.rgc_linear_forward_batch(n, _ptrs(Xs), _i64s(ldxs), _i64s(ks), _ptrs(Ws), _i64s(ldws), _i64s(ds),
                                        _ptrs(Ps) if Ps else None, _ptrs(Ys), _i64s(ds), _ptrs(XPs) if Ps else None,
                                        T, r, _stream(dev)))
    return Ys, XPs


def rgc_linear_backward(D: torch.Tensor, W: torch.Tensor, XP: torch.Tensor | None = None,
                        C: torch.Tensor | None = None, dX: torch.Tensor | None = None,
                        workspace: Workspace | None = None) -> torch.Tensor:
    """dX = bf16(D W); with XP and C also C += D^T XP (in place), in one call."""
    lib = load_library()
    if (XP is None) != (C is None):
        raise RgcError("give both XP and C, or neither")
    dev = _need_gpu(D, W, *([XP, C] if XP is not None else []))
    ldd = _rows(D, torch.bfloat16, "D")
    ldw = _rows(W, torch.bfloat16, "W")
    T, d = D.shape
    k = W.shape[1]
    if W.shape[0] != d:
        raise RgcError("W must be d x k with d = D.shape[1]")
    r = 0
    if XP is not None:
        _dense(XP, torch.bfloat16, "XP")
        _dense(C, torch.float32, "C")
        r = XP.shape[1]
        if XP.shape[0] != T or tuple(C.shape) != (d, r):
            raise RgcError("shapes must be XP: T x r, C: d x r")
    if dX is None:
        dX = torch.empty((T, k), dtype=torch.bfloat16, device=dev)
    lddx = _rows(dX, torch.bfloat16, "dX")
    ws = workspace or default_workspace(dev)
    wp, wn = ws.get(lib.rgc_linear_backward_workspace_size(T, d, k, r))
    _check(lib.rgc_linear_backward(D.data_ptr(), ldd, W.data_ptr(), ldw, XP.data_ptr() if XP is not None else None,
                                   C.data_ptr() if C is not None else None, dX.data_ptr(), lddx, T, d, k, r, wp, wn,
                                   _stream(dev)))
    return dX
