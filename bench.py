"""Benchmark of the sketch hot path on one MI355X.

The bench line is one training step of the full Qwen3-8B-shaped projection
set: 36 layers x 7 matrices (q and o 4096->4096, k and v 4096->1024, gate
and up 4096->12288, down 12288->4096; W is out x in), all 252 weight matrices
(12.9 GiB of bf16) resident in HBM, rank 128, QR-of-Gaussian projections
redrawn every step, 32768 tokens in 8 microbatches of 4096. Per layer:

  rgc_sample_projections (QR, the layer's 7 matrices in one batched call;
                          drawn one step ahead on a second stream)
  8 x (rgc_project_batch + rgc_accumulate_batch), each covering the 7 matrices
  rgc_apply_batch over the 7 matrices (tau = 1e-3)

Layers run one after another (layer-major). Inputs are synthetic and resident
in HBM before timing: one set of X ~ N(0,1) activations (shared by q/k/v and
by gate/up, as in the real block) and D ~ N(0, 1e-3^2) output gradients,
reused by every layer (a set is 4.2 GB, far above the 256 MB Infinity Cache,
and a layer reads it all between two reads of the same bytes); every layer
has its own W ~ N(0, 0.02^2), sketches and projections. Prints one JSON line.

--workload selects the other workload shapes (same fields).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

BLOCK_1P7B = [  # name, d (out), k (in), input activation
    ("q", 2048, 2048, "attn_in"), ("k", 1024, 2048, "attn_in"), ("v", 1024, 2048, "attn_in"),
    ("o", 2048, 2048, "attn_out"), ("gate", 6144, 2048, "mlp_in"), ("up", 6144, 2048, "mlp_in"),
    ("down", 2048, 6144, "mlp_act"),
]
LAYER_8B = [  # one layer of the Qwen3-8B-shaped projection set
    ("q", 4096, 4096, "attn_in"), ("k", 1024, 4096, "attn_in"), ("v", 1024, 4096, "attn_in"),
    ("o", 4096, 4096, "attn_out"), ("gate", 12288, 4096, "mlp_in"), ("up", 12288, 4096, "mlp_in"),
    ("down", 4096, 12288, "mlp_act"),
]
#   layers:  layers of the set, each with its own W, sketches and projections
#   refresh: a new projection every step (QR, drawn one step ahead); else drawn once (fixed Rademacher)
#   x_dist:  "normal" or "t4" (Student-t with 4 degrees of freedom scaled to unit variance)
WORKLOADS = {
    "qwen3-8b": {"desc": "qwen3-8b-shaped projection set, 36 layers x 7 matrices (12.9 GiB bf16 W resident), "
                         "r=128 QR redrawn every step, 32768 tokens in 8x4096",
                 "matrices": LAYER_8B, "layers": 36, "r": 128, "kind": "qr", "refresh": True, "tokens": 32768,
                 "microbatch": 4096, "tau": 1e-3, "x_dist": "normal", "cfg": 5},
    "qwen3-8b-layer": {"desc": "one layer of the qwen3-8b-shaped set (7 matrices), r=128 QR, 32768 tokens in 8x4096",
                       "matrices": LAYER_8B, "layers": 1, "r": 128, "kind": "qr", "refresh": True, "tokens": 32768,
                       "microbatch": 4096, "tau": 1e-3, "x_dist": "normal", "cfg": 5},
    "qwen3-1.7b-block": {"desc": "qwen3-1.7b-block 7 projections, r=64 QR, 32768 tokens in 8x4096",
                         "matrices": BLOCK_1P7B, "layers": 1, "r": 64, "kind": "qr", "refresh": True,
                         "tokens": 32768, "microbatch": 4096, "tau": 1e-3, "x_dist": "normal", "cfg": 2},
    "qwen3-1.7b-block-r256": {"desc": "qwen3-1.7b-block 7 projections, r=256 fixed Rademacher, 65536 tokens in "
                                      "16x4096", "matrices": BLOCK_1P7B, "layers": 1, "r": 256, "kind": "rademacher",
                              "refresh": False, "tokens": 65536, "microbatch": 4096, "tau": 1e-3,
                              "x_dist": "normal", "cfg": 3},
    "square-4096": {"desc": "square layer 4096x4096, r=64 QR new per update, 131072 tokens in 32x4096",
                    "matrices": [("w", 4096, 4096, "x")], "layers": 1, "r": 64, "kind": "qr", "refresh": True,
                    "tokens": 131072, "microbatch": 4096, "tau": 1e-3, "x_dist": "t4", "cfg": 4},
}
DEFAULT_WORKLOAD = "qwen3-8b"

# HBM traffic of the roofline kernel, measured with rocprofv3 counters; each
# record is used only while the sources it was taken from are unchanged.
TRAFFIC_RECORDS = {  # one layer of the 8B set launches exactly what each of the 36 does
    "qwen3-8b": "profiles/traffic_accumulate_qwen3_8b_r128.md",
    "qwen3-8b-layer": "profiles/traffic_accumulate_qwen3_8b_r128.md",
    "qwen3-1.7b-block": "profiles/traffic_accumulate_qwen3_1p7b_block_r64.md",
}
KERNEL_SOURCES = ["rank_randomized_gradient_amd/csrc/rgc_sketch.hip", "rank_randomized_gradient_amd/csrc/rgc_device.hpp",
                  "rank_randomized_gradient_amd/csrc/rgc_internal.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS),
                    help="the bench line is the default; the others measure the remaining workload shapes")
    ap.add_argument("--carried-norm", action="store_true",
                    help="the step applies with ||W|| carried from the previous update (rgc_apply_carried_batch: "
                         "W read once per apply); streamed from W once before the warm-up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--probe", choices=["shared-x", "linear", "sample"], default=None,
                    help="instead of the step: shared-x times rgc_project_shared against rgc_project_batch for the "
                         "workload's matrices that read one X; linear times the layer products with the sketch "
                         "attached (rgc_linear_forward / rgc_linear_backward) against torch's GEMM plus the "
                         "separate sketch call, per matrix of one layer (--steps calls each; with --steps 1, one "
                         "call each for counter runs); sample times one layer's projection sampling "
                         "(rgc_sample_projections) back to back; each prints one JSON line")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (a plain copy kernel of "
                         "known size, for calibrating the profiler's HBM byte counters)")
    return ap.parse_args()


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: its
    recording skips the system-scope release (an L2 writeback and invalidate)
    that a default event performs, which otherwise stalls the next kernel by
    ~10 us and so inflates per-call times measured between dependent launches.
    Created through the HIP runtime that torch has loaded (the same instance
    the library launches through)."""

    _rt = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence (timing stays enabled)

    @classmethod
    def runtime(cls):
        if cls._rt is None:
            import ctypes

            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            rt = ctypes.CDLL(path)
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._rt = rt
        return cls._rt

    def __init__(self):
        import ctypes

        self.ev = ctypes.c_void_p()
        if self.runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self.runtime().hipEventRecord(self.ev, ctypes_stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end) -> float:
        import ctypes

        ms = ctypes.c_float()
        if self.runtime().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self.ev and TimingEvent._rt is not None:
            TimingEvent._rt.hipEventDestroy(self.ev)


def ctypes_stream(stream):
    import ctypes

    return ctypes.c_void_p(stream.cuda_stream)


def sources_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (the accumulate's, or with key
    project_hbm_bytes_per_launch the project's) measured with rocprofv3
    counters (the record gives the commands and the copy-kernel scaling), or
    None when the record is missing or was taken from different kernel
    sources."""
    rel = TRAFFIC_RECORDS.get(workload)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    fields = {}
    with open(os.path.join(ROOT, rel)) as f:
        for line in f:
            if ":" in line and line.lstrip().startswith("- "):
                name, _, val = line.strip()[2:].partition(":")
                fields[name.strip()] = val.strip().strip("`")
    if fields.get("sources_sha256") != sources_digest():
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def step_seed(cfg: int, step: int, layer: int, m: int) -> int:
    return (cfg << 56) | ((step & 0xFFFFFFFF) << 24) | (layer << 8) | m


class Calls:
    """The library calls of one step, marshalled once: every call below is a
    ctypes call with argument arrays built up front (the seeds arrays are
    rewritten in place before each use). Validation still runs in the library
    on every call; only Python's per-call marshalling is hoisted."""

    def __init__(self, rgc, lib, wl, X, D, W, P_sets, C, XP, ws_main, ws_side, ws_acc, s_main, s_side):
        import torch

        self.rgc, self.lib = rgc, lib
        mats, r, mb = wl["matrices"], wl["r"], wl["microbatch"]
        n, L = len(mats), wl["layers"]
        self.n, self.L, self.n_mb = n, L, wl["tokens"] // mb
        i64, vp, u64, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_float
        arr = lambda t, vals: (t * len(vals))(*vals)  # noqa: E731
        self.kind = rgc.RGC_PROJ_QR_GAUSSIAN if wl["kind"] == "qr" else rgc.RGC_PROJ_RADEMACHER
        ks = [k for _, _, k, _ in mats]
        ds = [d for _, d, _, _ in mats]
        self.ks_arr, self.ds_arr = arr(i64, ks), arr(i64, ds)
        self.r, self.mb, self.tau = r, mb, float(wl["tau"])
        self.sm, self.ss = vp(s_main.cuda_stream), vp(s_side.cuda_stream)
        # workspaces: the largest query of any call on each stream
        need_main = max(lib.rgc_project_batch_workspace_size(n, self.ks_arr, mb, r),
                        lib.rgc_accumulate_batch_workspace_size(n, self.ds_arr, mb, r),
                        lib.rgc_apply_batch_workspace_size(n, self.ds_arr, self.ks_arr, r),
                        lib.rgc_sample_projections_workspace_size(self.kind, n, self.ks_arr, r))
        need_side = lib.rgc_sample_projections_workspace_size(self.kind, n, self.ks_arr, r)
        self.wm = (vp(ws_main.get(need_main)[0].value), need_main)
        # the accumulate's own workspace: it carries the split tiles' partial
        # sums from a layer's first microbatch to its last (deferred finish)
        need_acc = lib.rgc_accumulate_batch_workspace_size(n, self.ds_arr, mb, r)
        self.wa = (vp(ws_acc.get(need_acc)[0].value if need_acc else 0), need_acc)
        self.wsd = (vp(ws_side.get(need_side)[0].value), need_side) if need_side else (vp(0), 0)
        self.seeds = [arr(u64, [0] * n) for _ in range(L)]
        self.p_ptrs = [[arr(vp, [p.data_ptr() for p in P_sets[b][l]]) for l in range(L)] for b in range(len(P_sets))]
        self.w_ptrs = [arr(vp, [w.data_ptr() for w in W[l]]) for l in range(L)]
        self.ldw = arr(i64, ks)
        self.c_ptrs = [arr(vp, [c.data_ptr() for c in C[l]]) for l in range(L)]
        self.xp_ptrs = arr(vp, [x.data_ptr() for x in XP])
        self.x_ptrs, self.ldx, self.d_ptrs, self.ldd = [], None, [], None
        for i in range(self.n_mb):
            xs = [X[src][i * mb:(i + 1) * mb] for _, _, _, src in mats]
            dd = [D[m][i * mb:(i + 1) * mb] for m in range(n)]
            self.x_ptrs.append(arr(vp, [x.data_ptr() for x in xs]))
            self.d_ptrs.append(arr(vp, [x.data_ptr() for x in dd]))
            self.ldx = arr(i64, [x.stride(0) for x in xs])
            self.ldd = arr(i64, [x.stride(0) for x in dd])
        self.step_seeds = arr(u64, [0] * n)
        self.wnorm2 = [torch.zeros(n, dtype=torch.float64, device=X[mats[0][3]].device) for _ in range(L)]
        self.carried_fresh = [True] * L

    def sample(self, cfg, step, layer, pbuf, side):
        for m in range(self.n):
            self.seeds[layer][m] = step_seed(cfg, step, layer, m)
        ws, stream = (self.wsd, self.ss) if side else (self.wm, self.sm)
        self.rgc._check(self.lib.rgc_sample_projections(self.kind, self.n, self.seeds[layer], self.ks_arr, self.r,
                                                        self.p_ptrs[pbuf][layer], ws[0], ws[1], stream))

    def project(self, pbuf, layer, i):
        self.rgc._check(self.lib.rgc_project_batch(self.n, self.x_ptrs[i], self.ldx, self.ks_arr,
                                                   self.p_ptrs[pbuf][layer], self.xp_ptrs, self.mb, self.r,
                                                   self.wm[0], self.wm[1], self.sm))

    def accumulate(self, layer, i):
        # one accumulation per layer and step: the first microbatch writes the
        # split tiles' partial slots, the last adds them into C
        phase = (1 if i == 0 else 0) | (2 if i == self.n_mb - 1 else 0)
        self.rgc._check(self.lib.rgc_accumulate_batch_deferred(
            self.n, self.d_ptrs[i], self.ldd, self.ds_arr, self.xp_ptrs, self.c_ptrs[layer], self.mb, self.r,
            self.wa[0], self.wa[1], phase, self.sm))

    def apply(self, cfg, step, pbuf, layer, carried=False):
        for m in range(self.n):
            self.step_seeds[m] = step_seed(cfg, step, layer, m) ^ (1 << 23)
        if carried:
            fresh = 1 if self.carried_fresh[layer] else 0
            self.carried_fresh[layer] = False
            self.rgc._check(self.lib.rgc_apply_carried_batch(
                self.n, self.w_ptrs[layer], self.ldw, self.c_ptrs[layer], self.p_ptrs[pbuf][layer], self.ds_arr,
                self.ks_arr, self.r, ctypes.c_float(self.tau), self.step_seeds, None,
                ctypes.c_void_p(self.wnorm2[layer].data_ptr()), fresh, self.wm[0], self.wm[1], self.sm))
            return
        self.rgc._check(self.lib.rgc_apply_batch(self.n, self.w_ptrs[layer], self.ldw, self.c_ptrs[layer],
                                                 self.p_ptrs[pbuf][layer], self.ds_arr, self.ks_arr, self.r,
                                                 ctypes.c_float(self.tau), self.step_seeds, None, self.wm[0],
                                                 self.wm[1], self.sm))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (got --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from rank_randomized_gradient_amd import rgc

    lib = rgc.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    if args.probe == "linear":
        probe_linear(args, wl, rgc, torch, dev)
        return
    if args.probe == "shared-x":
        probe_shared_x(args, wl, rgc, torch, dev)
        return
    if args.probe == "sample":
        probe_sample(args, wl, rgc, torch, dev)
        return
    cfg, r, T, mb, L = wl["cfg"], wl["r"], wl["tokens"], wl["microbatch"], wl["layers"]
    n_mb = T // mb
    mats = wl["matrices"]
    n = len(mats)

    # ---- synthetic inputs, resident in HBM ------------------------------------
    g = torch.Generator(device=dev)
    g.manual_seed(2024)

    def normal(shape, std):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    def t4(shape):
        # Student-t, 4 degrees of freedom: Z / sqrt(chi2_4 / 4), scaled by 1/sqrt(2) to unit variance
        z = torch.randn(*shape, generator=g, device=dev)
        chi2 = sum(torch.randn(*shape, generator=g, device=dev) ** 2 for _ in range(4))
        return (z / torch.sqrt(chi2 / 4) / 2 ** 0.5).to(torch.bfloat16)

    acts = {}
    for _, _, k, src in mats:
        acts[src] = k
    X = {name: (t4((T, width)) if wl["x_dist"] == "t4" else normal((T, width), 1.0)) for name, width in acts.items()}
    D = [normal((T, d), 1e-3) for _, d, _, _ in mats]
    W = [[normal((d, k), 0.02) for _, d, k, _ in mats] for _ in range(L)]
    # two sets of projections (drawn one step ahead) per layer
    P_sets = [[[torch.empty((k, r), dtype=torch.bfloat16, device=dev) for _, _, k, _ in mats] for _ in range(L)]
              for _ in range(2 if wl["refresh"] else 1)]
    # each layer's 7 sketches are views of one buffer, so that zeroing them is one launch
    c_layer = [torch.zeros(sum(d for _, d, _, _ in mats) * r, dtype=torch.float32, device=dev) for _ in range(L)]
    C = []
    for l in range(L):
        views, off = [], 0
        for _, d, _, _ in mats:
            views.append(c_layer[l][off:off + d * r].view(d, r))
            off += d * r
        C.append(views)
    XP = [torch.empty((mb, r), dtype=torch.bfloat16, device=dev) for _ in mats]
    s_main = torch.cuda.current_stream(dev)
    s_side = torch.cuda.Stream(device=dev)  # default priority
    calls = Calls(rgc, lib, wl, X, D, W, P_sets, C, XP, rgc.Workspace(dev), rgc.Workspace(dev), rgc.Workspace(dev),
                  s_main, s_side)
    torch.cuda.synchronize()

    # The projections of step s depend only on their seeds, so they are drawn one
    # step ahead on the second stream, overlapping step s - 1; two sets of P
    # buffers, ordered by events. Every timed step still draws exactly one set
    # (the first timed step's set is drawn during the warm-up).
    ev_ready, ev_free = [None, None], [None, None]

    def draw_ahead(step):
        buf = step % 2
        with torch.cuda.stream(s_side):
            if ev_free[buf] is not None:
                s_side.wait_event(ev_free[buf])  # the step that last read this set is done
            for l in range(L):
                calls.sample(cfg, step, l, buf, side=True)
            ev = torch.cuda.Event()
            ev.record(s_side)
            ev_ready[buf] = ev

    if not wl["refresh"]:
        for l in range(L):
            calls.sample(cfg, 0, l, 0, side=False)  # a fixed projection, drawn once

    # Event pairs around calls, when timing inside steps. An event recorded
    # between two dependent launches delays the second by several us (its
    # packet, even without a system fence), so a call's time inside steps is
    # taken as a difference of brackets that each hold one such delay: pass
    # "single" brackets every call alone, pass "pairs" every project with the
    # accumulate that follows it, pass "tail" every layer's last accumulate
    # with the apply that follows it. Then accumulate = pair - project alone,
    # project = pair - accumulate alone, apply = tail - accumulate alone.
    pairs = {k: [] for k in ("project", "accumulate", "accumulate_last", "apply", "pair", "tail")}

    def bracket(name, *fns, also=None):
        a, b = TimingEvent(), TimingEvent()
        a.record(s_main)
        for fn in fns:
            fn()
        b.record(s_main)
        pairs[name].append((a, b))
        if also:
            pairs[also].append((a, b))

    def one_step(step, mode=None):
        buf = 0
        if wl["refresh"]:
            buf = step % 2
            if ev_ready[buf] is None:
                draw_ahead(step)
            s_main.wait_event(ev_ready[buf])
            ev_ready[buf] = None
            draw_ahead(step + 1)
        for l in range(L):
            c_layer[l].zero_()
            for i in range(n_mb):
                prj = lambda: calls.project(buf, l, i)  # noqa: E731
                acc = lambda: calls.accumulate(l, i)  # noqa: E731
                if mode == "single":
                    bracket("project", prj)
                    bracket("accumulate", acc, also="accumulate_last" if i == n_mb - 1 else None)
                elif mode == "pairs":
                    bracket("pair", prj, acc)
                elif mode == "tail" and i == n_mb - 1:
                    prj()
                else:
                    prj()
                    acc()
            app = lambda: calls.apply(cfg, step, buf, l, args.carried_norm)  # noqa: E731
            if mode == "single":
                bracket("apply", app)
            elif mode == "tail":
                bracket("tail", lambda: calls.accumulate(l, n_mb - 1), app)
            else:
                app()
        if wl["refresh"]:
            ev = torch.cuda.Event()
            ev.record(s_main)
            ev_free[buf] = ev

    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ------------------------------------------
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        one_step(args.warmup + s)
    s_main.wait_stream(s_side)  # the last draw ends inside the timed region
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    tokens_per_s = T / (ms_per_step / 1e3)
    base = args.warmup + args.steps

    # the spread of single steps (a second pass, an event pair around each step)
    single = []
    for s in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        one_step(base + s)
        s_main.wait_stream(s_side)
        b.record()
        torch.cuda.synchronize()
        single.append(a.elapsed_time(b))
    single.sort()
    step_spread = {"min": round(single[0], 4), "median": round(single[len(single) // 2], 4),
                   "max": round(single[-1], 4)}
    base += args.steps

    # algorithmic work per launch (bytes and flops), per entry point
    acc_bytes = sum(2 * mb * d + 2 * mb * r + 8 * d * r for _, d, _, _ in mats)
    acc_flops = sum(2 * mb * d * r for _, d, _, _ in mats)
    prj_bytes = sum(2 * mb * k + 2 * mb * r + 2 * k * r for _, _, k, _ in mats)
    prj_flops = sum(2 * mb * k * r for _, _, k, _ in mats)
    app_bytes = sum(6 * d * k + 8 * d * r + 4 * k * r for _, d, k, _ in mats)
    appc_bytes = sum(4 * d * k + 8 * d * r + 4 * k * r for _, d, k, _ in mats)  # W read once
    smp_bytes = sum(2 * k * r for _, _, k, _ in mats)
    app_launch_bytes = appc_bytes if args.carried_norm else app_bytes

    # each call's duration inside steps: three more passes of K steps like the
    # timed ones, with event pairs on the launch stream (timing-only events
    # without a system-scope fence) around calls or pairs of calls (above)
    kern, in_step = {}, {}
    if not args.no_kernel_timing:
        for mode in ("single", "pairs", "tail"):
            torch.cuda.synchronize()
            for s in range(args.steps):
                one_step(base + s, mode)
            s_main.wait_stream(s_side)
            torch.cuda.synchronize()
            base += args.steps
        mean = {name: sum(a.elapsed_ms(b) for a, b in prs) * 1e-3 / len(prs) for name, prs in pairs.items()}
        in_step = {"accumulate": mean["pair"] - mean["project"], "project": mean["pair"] - mean["accumulate"],
                   "apply": mean["tail"] - mean["accumulate_last"]}  # seconds per call

        # Per-entry-point timing back to back: HIP events on the launch stream
        # around K repetitions of one step's calls of a single entry point.
        def time_op(fn):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for s in range(args.steps):
                fn(s)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e-3 / args.steps  # seconds per step

        per_step = {
            "sample_projection": time_op(lambda s: [calls.sample(cfg, base + s, l, 0, side=False) for l in range(L)]),
            "project": time_op(lambda s: [calls.project(0, l, i) for l in range(L) for i in range(n_mb)]),
            "accumulate": time_op(lambda s: [calls.accumulate(l, i) for l in range(L) for i in range(n_mb)]),
            "apply": time_op(lambda s: [calls.apply(cfg, base + s, 0, l, args.carried_norm) for l in range(L)]),
        }
        if not args.carried_norm:
            for l in range(L):
                calls.apply(cfg, base, 0, l, carried=True)  # the first call streams ||W||; the timed ones carry it
        per_step["apply_carried"] = time_op(lambda s: [calls.apply(cfg, base + s, 0, l, True) for l in range(L)])
        launches = {"project": L * n_mb, "accumulate": L * n_mb, "apply": L, "apply_carried": L,
                    "sample_projection": L}
        work = {"project": (prj_bytes, prj_flops), "accumulate": (acc_bytes, acc_flops),
                "apply": (app_launch_bytes, 0), "apply_carried": (appc_bytes, 0), "sample_projection": (smp_bytes, 0)}
        # A difference of brackets can come out far below the back-to-back
        # duration when something else stretches the brackets unevenly (a
        # profiler that intercepts each dispatch does); a launch cannot run
        # much faster inside a step than back to back, so such an estimate is
        # dropped for the back-to-back mean and the entry says so.
        rejected = []
        for name in list(in_step):
            b2b = per_step[name] / launches[name]
            if in_step[name] < 0.8 * b2b:
                rejected.append(name)
                in_step[name] = b2b
        for name, sps in per_step.items():
            by, fl = work[name]
            avg = sps / launches[name]
            e = {"launches_per_step": launches[name], "avg_us": 1e6 * avg, "GBs": by / avg / 1e9}
            if fl:
                e["TFLOPs"] = fl / avg / 1e12
            if name in in_step:
                t = in_step[name]
                e.update({"avg_us_in_step": 1e6 * t, "GBs_in_step": by / t / 1e9})
                if name in rejected:
                    e["in_step_estimate"] = "rejected (below 0.8 x back to back); back-to-back mean used"
                if fl:
                    e["TFLOPs_in_step"] = fl / t / 1e12
                    ai = fl / by
                    bound = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
                    e["arith_intensity"] = ai
                    e["frac_bounding_roofline_in_step"] = (fl / t / 1e12) / bound
            e["hbm_frac"] = e.get("GBs_in_step", e["GBs"]) / HBM_PEAK_GBS
            kern[name] = e
        if not wl["refresh"]:
            kern["sample_projection"]["launches_per_step"] = 0

    # dominant kernel: the entry point with the most time inside a step.
    # achieved = algorithmic bytes per launch / the launch's mean duration inside steps
    roofline = None
    if in_step:
        share = {nm: in_step[nm] * (L * n_mb if nm != "apply" else L) for nm in in_step}
        dom = max(share, key=share.get)
        by, fl = work[dom]
        t = in_step[dom]
        kernels = {"accumulate": f"rgc_accumulate_batch_deferred (accumulate_kernel<{r}> per call + "
                                 f"finish_tiles_kernel<{r},false> on a layer's last of {n_mb} calls)",
                   "project": f"rgc_project_batch (project_kernel<{r}> + finish_tiles_kernel<{r},true>)",
                   "apply": "rgc_apply_batch (norms, scale, update launches)"}
        achieved = by / t / 1e9
        roofline = {"kernel": kernels[dom], "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "launch_us_in_step": round(1e6 * t, 2),
                    "launch_time_from": ("back-to-back mean (in-step estimate rejected)" if dom in rejected
                                         else "in-step: difference of event-bracketed passes"),
                    "traffic": (recorded_traffic(args.workload) if dom == "accumulate" else
                                recorded_traffic(args.workload, "project_hbm_bytes_per_launch")
                                if dom == "project" else None),
                    "algorithmic_bytes_per_launch": by,
                    "step_time_share": round(share[dom] / (ms_per_step * 1e-3), 4)}
        if fl:
            roofline["arith_intensity_flop_per_byte"] = round(fl / by, 1)

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline and args.workload == DEFAULT_WORKLOAD:
        cpu = cpu_baseline(X, D, W[0], mats, wl)

    acc = kern.get("accumulate", {})
    app = kern.get("apply", {})
    out = {
        "metric": "sketch-accumulate TFLOP/s + fused-apply HBM GB/s (% roofline), tokens/s/step",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "single_step_ms": step_spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "layers": L, "matrices_per_layer": n, "r": r, "tokens_per_step": T,
                   "microbatch": mb, "projection": "qr-gaussian" if wl["kind"] == "qr" else "rademacher, fixed",
                   "tau": wl["tau"],
                   "accumulation": f"deferred: split-tile partials summed into C once per layer and step "
                                   f"(after the last of {n_mb} microbatches)",
                   "weight_norm": "carried from the previous update" if args.carried_norm else "streamed from W",
                   "resident_weight_GiB": round(sum(w.numel() * 2 for ws_ in W for w in ws_) / 2**30, 2)},
        "sketch_accumulate_TFLOPs": round(acc["TFLOPs_in_step"], 2) if acc else None,
        "sketch_accumulate_frac_bf16_peak": round(acc["TFLOPs_in_step"] / BF16_PEAK_TFLOPS, 4) if acc else None,
        "sketch_accumulate_frac_bounding_roofline": round(acc["frac_bounding_roofline_in_step"], 4) if acc else None,
        "fused_apply_GBs": round(app["GBs_in_step"], 1) if app else None,
        "fused_apply_frac_hbm_peak": round(app["GBs_in_step"] / HBM_PEAK_GBS, 4) if app else None,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kern.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def probe_shared_x(args, wl, rgc, torch, dev):
    """One microbatch of the workload's matrices that read one X (q/k/v,
    gate/up): rgc_project_shared (X read once per group, up to 256 ranks a
    group) against rgc_project_batch of the same matrices (X read once per
    matrix). Times are HIP event pairs around --steps calls of each."""
    r, mb, mats = wl["r"], wl["microbatch"], wl["matrices"]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    groups = {}
    for m, (_, _, k, src) in enumerate(mats):
        groups.setdefault(src, []).append(m)
    cap = max(1, min(4, 256 // r))
    out = {"probe": "shared-x", "workload": wl["desc"], "r": r, "tokens": mb, "groups": []}
    for src, members in groups.items():
        if len(members) < 2:
            continue
        members = members[:cap]
        k = mats[members[0]][2]
        x = torch.randn(mb, k, generator=g, device=dev).to(torch.bfloat16)
        ps = [(torch.randn(k, r, generator=g, device=dev) * 0.1).to(torch.bfloat16) for _ in members]
        xps = [torch.empty(mb, r, dtype=torch.bfloat16, device=dev) for _ in members]
        ws = rgc.Workspace(dev)
        shared = lambda: rgc.rgc_project_shared(x, ps, outs=xps, workspace=ws)  # noqa: E731
        batch = lambda: rgc.rgc_project_batch([x] * len(ps), ps, outs=xps, workspace=ws)  # noqa: E731
        times = {}
        for name, fn in (("shared", shared), ("batch", batch)):
            if args.steps > 1:
                for _ in range(3):
                    fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            times[name] = round(a.elapsed_time(b) * 1e3 / args.steps, 2)
        out["groups"].append({"input": src, "matrices": [mats[m][0] for m in members], "k": k,
                              "unique_x_MB": round(2 * mb * k / 1e6, 1), "shared_us": times["shared"],
                              "batch_us": times["batch"]})
    if args.copy_mib > 0:
        src_t = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src_t).copy_(src_t)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def probe_sample(args, wl, rgc, torch, dev):
    """The projection sampling of one layer of the workload alone: one
    rgc_sample_projections call over the layer's matrices (the QR chain, or
    the Rademacher draw), --steps calls back to back with fresh seeds, timed
    with a HIP event pair; under rocprofv3 it gives the chain's kernel split."""
    r, mats = wl["r"], wl["matrices"]
    kind = "qr" if wl["kind"] == "qr" else "rademacher"
    ps = [torch.empty((k, r), dtype=torch.bfloat16, device=dev) for _, _, k, _ in mats]
    ws = rgc.Workspace(dev)
    for i in range(3):
        rgc.rgc_sample_projections(kind, [i * len(mats) + m for m in range(len(mats))], ps, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        rgc.rgc_sample_projections(kind, [((i + 3) << 8) + m for m in range(len(mats))], ps, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    out = {"probe": "sample", "workload": wl["desc"], "kind": kind, "r": r, "matrices": len(mats),
           "ks": [k for _, _, k, _ in mats], "calls": args.steps,
           "us_per_call": round(a.elapsed_time(b) * 1e3 / args.steps, 2)}
    print(json.dumps(out), flush=True)


def probe_linear(args, wl, rgc, torch, dev):
    """One microbatch through each matrix of one layer of the workload: the
    forward [Y | XP] = X [W^T | P] as one rgc_linear_forward call against
    torch's Y = X W^T (hipBLASLt) followed by rgc_project, and the backward
    dX = D W with C += D^T XP as one rgc_linear_backward call against torch's
    D W followed by rgc_accumulate; also the library's Y and dX alone (r = 0).
    Times are HIP event pairs on the current stream around --steps calls."""
    r, mb, mats = wl["r"], wl["microbatch"], wl["matrices"]
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    ws = rgc.Workspace(dev)
    out = {"probe": "linear", "workload": wl["desc"], "r": r, "tokens": mb, "matrices": []}

    def timed(fn):
        if args.steps > 1:
            for _ in range(2):
                fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / args.steps

    tot = {}
    for name, d, k, _ in mats:
        x = torch.randn(mb, k, generator=g, device=dev).to(torch.bfloat16)
        w = (torch.randn(d, k, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        p = (torch.randn(k, r, generator=g, device=dev) / r ** 0.5).to(torch.bfloat16)
        dd = (torch.randn(mb, d, generator=g, device=dev) * 1e-3).to(torch.bfloat16)
        y = torch.empty(mb, d, dtype=torch.bfloat16, device=dev)
        xp = torch.empty(mb, r, dtype=torch.bfloat16, device=dev)
        dx = torch.empty(mb, k, dtype=torch.bfloat16, device=dev)
        c = torch.zeros(d, r, device=dev)
        flops = 2.0 * mb * d * k
        t = {
            "fwd_fused_us": timed(lambda: rgc.rgc_linear_forward(x, w, p, Y=y, XP=xp)),
            "fwd_torch_plus_project_us": timed(lambda: (torch.matmul(x, w.t(), out=y),
                                                        rgc.rgc_project(x, p, out=xp, workspace=ws))),
            "fwd_lib_gemm_us": timed(lambda: rgc.rgc_linear_forward(x, w, Y=y)),
            "fwd_torch_gemm_us": timed(lambda: torch.matmul(x, w.t(), out=y)),
            "bwd_fused_us": timed(lambda: rgc.rgc_linear_backward(dd, w, xp, c, dX=dx, workspace=ws)),
            "bwd_torch_plus_accumulate_us": timed(lambda: (torch.matmul(dd, w, out=dx),
                                                           rgc.rgc_accumulate(dd, xp, c, workspace=ws))),
            "bwd_lib_gemm_us": timed(lambda: rgc.rgc_linear_backward(dd, w, dX=dx)),
            "bwd_torch_gemm_us": timed(lambda: torch.matmul(dd, w, out=dx)),
        }
        for key, v in t.items():
            tot[key] = tot.get(key, 0.0) + v
        row = {"matrix": name, "d": d, "k": k}
        row.update({key: round(v, 2) for key, v in t.items()})
        row["lib_gemm_TFLOPs"] = round(flops / t["fwd_lib_gemm_us"] / 1e6, 1)
        row["torch_gemm_TFLOPs"] = round(flops / t["fwd_torch_gemm_us"] / 1e6, 1)
        out["matrices"].append(row)
    out["layer_total_us"] = {key: round(v, 1) for key, v in tot.items()}
    # the matrices that read one X, as one batched launch each (a block's q, k,
    # v; gate and up) against torch's separate GEMMs plus rgc_project_batch
    groups = {}
    for m, (_, _, _, src) in enumerate(mats):
        groups.setdefault(src, []).append(m)
    out["shared_input_batches"] = []
    for src, members in groups.items():
        if len(members) < 2:
            continue
        k = mats[members[0]][2]
        x = torch.randn(mb, k, generator=g, device=dev).to(torch.bfloat16)
        ws_ = [(torch.randn(mats[m][1], k, generator=g, device=dev) * 0.02).to(torch.bfloat16) for m in members]
        ps = [(torch.randn(k, r, generator=g, device=dev) / r ** 0.5).to(torch.bfloat16) for _ in members]
        ys = [torch.empty(mb, mats[m][1], dtype=torch.bfloat16, device=dev) for m in members]
        xps = [torch.empty(mb, r, dtype=torch.bfloat16, device=dev) for _ in members]

        def torch_fwd():
            for w_, y_ in zip(ws_, ys):
                torch.matmul(x, w_.t(), out=y_)
            rgc.rgc_project_batch([x] * len(ps), ps, outs=xps, workspace=ws)

        out["shared_input_batches"].append({
            "input": src, "matrices": [mats[m][0] for m in members],
            "fwd_fused_batch_us": round(timed(lambda: rgc.rgc_linear_forward_batch([x] * len(ps), ws_, ps)), 2),
            "fwd_torch_plus_project_batch_us": round(timed(torch_fwd), 2)})
    if args.copy_mib > 0:
        src_t = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src_t).copy_(src_t)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _blas() -> tuple[str, int]:
    try:
        from threadpoolctl import threadpool_info

        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            return f"{i.get('internal_api', '?')} {i.get('version', '')}".strip(), int(i.get("num_threads", 1))
    except Exception:
        pass
    return "unknown", len(os.sched_getaffinity(0))


def cpu_baseline(X, D, W, mats, wl):
    """The CPU oracle, untuned, on a bounded sample of the same workload: one
    full layer (about 15 s of CPU work): the layer's 7 QR projections, every
    4096-token microbatch of project + accumulate for its 7 matrices, and the
    updates of all 7 matrices. The step time is that layer's time x the
    number of layers (labelled as an extrapolation)."""
    import numpy as np

    import oracle as orc
    from rank_randomized_gradient_amd import synth

    r, mb, L = wl["r"], wl["microbatch"], wl["layers"]
    n_mb = wl["tokens"] // mb
    bits = synth.to_numpy_bits
    t0 = time.perf_counter()
    ps = [orc.qr_projection(step_seed(wl["cfg"], 0, 0, m), k, r) for m, (_, _, k, _) in enumerate(mats)]
    t1 = time.perf_counter()
    cs = [np.zeros((d, r), np.float32) for _, d, _, _ in mats]
    t_mb = 0.0
    for i in range(n_mb):
        xs = {name: bits(x[i * mb:(i + 1) * mb]) for name, x in X.items()}  # host copies, not timed
        ds = [bits(d[i * mb:(i + 1) * mb]) for d in D]
        ta = time.perf_counter()
        for m, (_, d, k, src) in enumerate(mats):
            cs[m] = orc.accumulate(cs[m], ds[m], orc.project(xs[src], ps[m]))
        t_mb += time.perf_counter() - ta
    t2 = time.perf_counter()
    for m in range(len(mats)):
        orc.apply_update(bits(W[m]), cs[m], ps[m], wl["tau"], step_seed(wl["cfg"], 0, 0, m))
    t3 = time.perf_counter()
    layer_s = (t1 - t0) + t_mb + (t3 - t2)
    step_s = L * layer_s
    # the contractions' flops in the sample: project and accumulate per microbatch, H = C P^T per update
    flops = sum(n_mb * (2 * mb * k * r + 2 * mb * d * r) + 2 * d * k * r for _, d, k, _ in mats)
    blas, threads = _blas()
    return {"value": round(wl["tokens"] / step_s, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "blas": blas, "gflops": round(flops / layer_s / 1e9, 2),
            "sample": f"one full layer: 7 QR projections ({t1 - t0:.1f}s) + {n_mb} microbatches of "
                      f"project+accumulate for 7 matrices ({t_mb:.1f}s) + the updates of all 7 matrices "
                      f"({t3 - t2:.1f}s) = {layer_s:.1f}s; step = {L} x that layer = {step_s:.0f}s "
                      f"(extrapolated x{L} layers)"}


if __name__ == "__main__":
    main()
