"""Benchmark of the sketch hot path on one MI355X.

One step = the whole path for one training step of one Qwen3-1.7B-shaped
block (q 2048->2048, k and v 2048->1024, o 2048->2048, gate and up
2048->6144, down 6144->2048; W is out x in), rank 64, QR-of-Gaussian
projections redrawn every step, 32768 tokens in 8 microbatches of 4096:

  rgc_sample_projections (QR, the 7 matrices in one batched call)
  8 x (rgc_project_batch + rgc_accumulate_batch), each covering the 7 matrices
  rgc_apply_batch over the 7 matrices (tau = 1e-3)

Inputs are synthetic and resident in HBM before timing: X ~ N(0,1) (shared by
q/k/v and by gate/up, as in the real block), D ~ N(0, 1e-3^2), W ~ N(0, 0.02^2),
all bf16. Prints one JSON line (see the fields below).
"""
from __future__ import annotations

import argparse
import json
import os
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
# The default is the bench line; the others measure the remaining workload shapes (same fields, their own name).
#   refresh: a new projection every step (QR, drawn inside the timed step); else drawn once (fixed Rademacher)
#   x_dist:  "normal" or "t4" (Student-t with 4 degrees of freedom scaled to unit variance)
WORKLOADS = {
    "qwen3-1.7b-block": {"desc": "qwen3-1.7b-block 7 projections, r=64 QR, 32768 tokens in 8x4096",
                         "matrices": BLOCK_1P7B, "r": 64, "kind": "qr", "refresh": True, "tokens": 32768,
                         "microbatch": 4096, "tau": 1e-3, "x_dist": "normal"},
    "qwen3-1.7b-block-r256": {"desc": "qwen3-1.7b-block 7 projections, r=256 fixed Rademacher, 65536 tokens in 16x4096",
                              "matrices": BLOCK_1P7B, "r": 256, "kind": "rademacher", "refresh": False,
                              "tokens": 65536, "microbatch": 4096, "tau": 1e-3, "x_dist": "normal"},
    "square-4096": {"desc": "square layer 4096x4096, r=64 QR new per update, 131072 tokens in 32x4096",
                    "matrices": [("w", 4096, 4096, "x")], "r": 64, "kind": "qr", "refresh": True, "tokens": 131072,
                    "microbatch": 4096, "tau": 1e-3, "x_dist": "t4"},
    "qwen3-8b-layer": {"desc": "one qwen3-8b-shaped layer (7 projections), r=128 QR, 32768 tokens in 8x4096",
                       "matrices": LAYER_8B, "r": 128, "kind": "qr", "refresh": True, "tokens": 32768,
                       "microbatch": 4096, "tau": 1e-3, "x_dist": "normal"},
}
WORKLOAD = WORKLOADS["qwen3-1.7b-block"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3-1.7b-block", choices=sorted(WORKLOADS),
                    help="the bench line is the default; the others measure the remaining workload shapes")
    ap.add_argument("--carried-norm", action="store_true",
                    help="the step applies with ||W|| carried from the previous update (rgc_apply_carried_batch: "
                         "W read once per apply); streamed from W once before the warm-up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (a plain copy kernel of "
                         "known size, for calibrating the profiler's HBM byte counters)")
    return ap.parse_args()


# Sources the accumulate kernel is built from; the HBM traffic recorded from
# profiler counters is reported only while they are unchanged.
KERNEL_SOURCES = ["rank_randomized_gradient_amd/csrc/rgc_sketch.hip", "rank_randomized_gradient_amd/csrc/rgc_device.hpp",
                  "rank_randomized_gradient_amd/csrc/rgc_internal.hpp"]
TRAFFIC_RECORD = "profiles/traffic_accumulate_qwen3_1p7b_block_r64.md"


def sources_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per accumulate launch measured with rocprofv3 counters (see the
    record for the commands and the copy-kernel scaling), or None when the
    record is missing or was taken from different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_RECORD)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.lstrip().startswith("- "):
                key, _, val = line.strip()[2:].partition(":")
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("sources_sha256") != sources_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_seed(step: int, m: int) -> int:
    return (2 << 32) | (step << 8) | m


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from rank_randomized_gradient_amd import rgc

    rgc.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    default_wl = args.workload == "qwen3-1.7b-block"
    r, T, mb = wl["r"], wl["tokens"], wl["microbatch"]
    n_mb = T // mb
    mats = wl["matrices"]

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
    W = [normal((d, k), 0.02) for _, d, k, _ in mats]
    P = [torch.empty((k, r), dtype=torch.bfloat16, device=dev) for _, _, k, _ in mats]
    # the 7 sketches are views of one buffer, so that zeroing them is one launch
    c_all = torch.zeros(sum(d for _, d, _, _ in mats) * r, dtype=torch.float32, device=dev)
    C, off = [], 0
    for _, d, _, _ in mats:
        C.append(c_all[off:off + d * r].view(d, r))
        off += d * r
    XP = [torch.empty((mb, r), dtype=torch.bfloat16, device=dev) for _ in mats]
    ws = rgc.Workspace(dev)
    torch.cuda.synchronize()

    # The projections of step s depend only on their seeds, so they are drawn one
    # step ahead on a second stream (default priority), overlapping step s - 1;
    # two sets of P buffers, ordered by events. Every timed step still draws
    # exactly one set (the first timed step's set is drawn during the warm-up).
    s_main = torch.cuda.current_stream(dev)
    s_side = torch.cuda.Stream(device=dev)
    ws_side = rgc.Workspace(dev)
    Pb = [P, [torch.empty_like(p) for p in P]]
    ev_ready, ev_free = [None, None], [None, None]

    def sample_all(step, Ps=None, workspace=None):
        # all projections of the block in one batched call (same bits as one call per matrix)
        rgc.rgc_sample_projections(wl["kind"], [step_seed(step, m) for m in range(len(mats))],
                                   Ps if Ps is not None else P, workspace=workspace or ws)

    def draw_ahead(step):
        buf = step % 2
        with torch.cuda.stream(s_side):
            if ev_free[buf] is not None:
                s_side.wait_event(ev_free[buf])  # the step that last read this set is done
            sample_all(step, Pb[buf], ws_side)
            ev = torch.cuda.Event()
            ev.record(s_side)
            ev_ready[buf] = ev

    if not wl["refresh"]:
        sample_all(0)  # a fixed projection, drawn once

    def project_mb(i, Ps=None):
        # the 7 projections of microbatch i in one launch (q/k/v and gate/up share their X)
        rgc.rgc_project_batch([X[src][i * mb:(i + 1) * mb] for _, _, _, src in mats], Ps if Ps is not None else P,
                              outs=XP, workspace=ws)

    def accumulate_mb(i):
        rgc.rgc_accumulate_batch([D[m][i * mb:(i + 1) * mb] for m in range(len(mats))], XP, C, workspace=ws)

    wnorm2 = torch.zeros(len(mats), dtype=torch.float64, device=dev)
    carried = {"fresh": True}

    def apply_carried(step, Ps=None):
        # the 7 updates with ||W||^2 carried in wnorm2 (streamed from W on the first call)
        rgc.rgc_apply_carried_batch(W, C, Ps if Ps is not None else P, wl["tau"],
                                    [step_seed(step, m) for m in range(len(mats))], wnorm2,
                                    fresh=carried["fresh"], workspace=ws)
        carried["fresh"] = False

    def apply_all(step, Ps=None):
        if args.carried_norm:
            apply_carried(step, Ps)
            return
        # the 7 updates in one batched call (norms sweep, step scalars, update sweep)
        rgc.rgc_apply_batch(W, C, Ps if Ps is not None else P, wl["tau"],
                            [step_seed(step, m) for m in range(len(mats))], workspace=ws)

    acc_pairs = []  # (start, end) events around accumulate calls, when timing them inside steps

    def one_step(step, time_accumulate=False):
        Ps = P
        if wl["refresh"]:
            buf = step % 2
            if ev_ready[buf] is None:
                draw_ahead(step)
            s_main.wait_event(ev_ready[buf])
            ev_ready[buf] = None
            draw_ahead(step + 1)
            Ps = Pb[buf]
        c_all.zero_()
        for i in range(n_mb):
            project_mb(i, Ps)
            if time_accumulate:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                accumulate_mb(i)
                b.record()
                acc_pairs.append((a, b))
            else:
                accumulate_mb(i)
        apply_all(step, Ps)
        if wl["refresh"]:
            ev = torch.cuda.Event()
            ev.record(s_main)
            ev_free[step % 2] = ev

    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ------------------------------------------
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        one_step(args.warmup + s)
    torch.cuda.current_stream(dev).wait_stream(s_side)  # the last draw ends inside the timed region
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    tokens_per_s = T / (ms_per_step / 1e3)

    # the spread of single steps (a second pass, an event pair around each step)
    single = []
    for s in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        one_step(args.warmup + args.steps + s)
        torch.cuda.current_stream(dev).wait_stream(s_side)
        b.record()
        torch.cuda.synchronize()
        single.append(a.elapsed_time(b))
    single.sort()
    step_spread = {"min": round(single[0], 4), "median": round(single[len(single) // 2], 4),
                   "max": round(single[-1], 4)}

    # the accumulate's duration inside steps (the roofline's kernel): a third pass
    # of K steps like the timed ones, with an event pair on the launch stream
    # around each rgc_accumulate_batch call
    acc_in_step_s = None
    if not args.no_kernel_timing:
        torch.cuda.synchronize()
        for s in range(args.steps):
            one_step(args.warmup + 2 * args.steps + s, time_accumulate=True)
        torch.cuda.current_stream(dev).wait_stream(s_side)
        torch.cuda.synchronize()
        acc_in_step_s = sum(a.elapsed_time(b) for a, b in acc_pairs) * 1e-3 / len(acc_pairs)

    # ---- per-entry-point timing ---------------------------------------------------
    # HIP events on the launch stream around K repetitions of one step's calls of
    # a single entry point, issued back to back (an event pair around every
    # microsecond-scale launch would time the event packets, not the kernels).
    kern = {}
    if not args.no_kernel_timing:
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
            "sample_projection": time_op(lambda s: sample_all(s)),
            "project": time_op(lambda s: [project_mb(i) for i in range(n_mb)]),
            "accumulate": time_op(lambda s: [accumulate_mb(i) for i in range(n_mb)]),
            "apply": time_op(lambda s: apply_all(s)),
        }
        if not args.carried_norm:
            apply_carried(0)  # the first call streams ||W||; the timed ones carry it
        per_step["apply_carried"] = time_op(lambda s: apply_carried(s))
        # algorithmic work per step (bytes and flops), per entry point
        acc_bytes = sum(2 * mb * d + 2 * mb * r + 8 * d * r for _, d, _, _ in mats) * n_mb
        acc_flops = sum(2 * mb * d * r for _, d, _, _ in mats) * n_mb
        prj_bytes = sum(2 * mb * k + 2 * mb * r + 2 * k * r for _, _, k, _ in mats) * n_mb
        prj_flops = sum(2 * mb * k * r for _, _, k, _ in mats) * n_mb
        app_bytes = sum(6 * d * k + 8 * d * r + 4 * k * r for _, d, k, _ in mats)
        appc_bytes = sum(4 * d * k + 8 * d * r + 4 * k * r for _, d, k, _ in mats)  # W read once
        smp_bytes = sum(2 * k * r for _, _, k, _ in mats)
        kern = {
            "accumulate": {"s_per_step": per_step["accumulate"], "launches_per_step": n_mb,
                           "avg_us": 1e6 * per_step["accumulate"] / n_mb,
                           "avg_us_in_step": 1e6 * acc_in_step_s,
                           "GBs_in_step": acc_bytes / n_mb / acc_in_step_s / 1e9,
                           "TFLOPs_in_step": acc_flops / n_mb / acc_in_step_s / 1e12,
                           "GBs": acc_bytes / per_step["accumulate"] / 1e9,
                           "TFLOPs": acc_flops / per_step["accumulate"] / 1e12},
            "project": {"s_per_step": per_step["project"], "launches_per_step": n_mb,
                        "avg_us": 1e6 * per_step["project"] / n_mb,
                        "GBs": prj_bytes / per_step["project"] / 1e9,
                        "TFLOPs": prj_flops / per_step["project"] / 1e12},
            "apply": {"s_per_step": per_step["apply"], "launches_per_step": 1,
                      "avg_us": 1e6 * per_step["apply"],
                      "GBs": (appc_bytes if args.carried_norm else app_bytes) / per_step["apply"] / 1e9},
            "apply_carried": {"s_per_step": per_step["apply_carried"], "launches_per_step": 1,
                              "avg_us": 1e6 * per_step["apply_carried"],
                              "GBs": appc_bytes / per_step["apply_carried"] / 1e9},
            "sample_projection": {"s_per_step": per_step["sample_projection"],
                                  "launches_per_step": 1 if wl["refresh"] else 0,
                                  "avg_us": 1e6 * per_step["sample_projection"],
                                  "GBs": smp_bytes / per_step["sample_projection"] / 1e9},
        }
        for v in kern.values():
            v["hbm_frac"] = v["GBs"] / HBM_PEAK_GBS
        kern["accumulate"]["mfma_frac"] = kern["accumulate"]["TFLOPs"] / BF16_PEAK_TFLOPS
        kern["project"]["mfma_frac"] = kern["project"]["TFLOPs"] / BF16_PEAK_TFLOPS

    # dominant kernel: the accumulate (the metric's named contraction); HBM-bound at r = 64.
    # achieved = algorithmic bytes per launch / the launch's mean duration inside the steps
    roofline = None
    if kern:
        achieved = acc_bytes / n_mb / acc_in_step_s / 1e9
        roofline = {"kernel": f"rgc_accumulate_batch (accumulate_kernel<{r}> + finish_tiles_kernel<{r},false>)",
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "launch_us_in_step": round(1e6 * acc_in_step_s, 2),
                    "traffic": recorded_traffic() if default_wl else None,
                    "algorithmic_bytes_per_launch": acc_bytes // n_mb}

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline and default_wl:
        cpu = cpu_baseline(X, D, W, mats, wl)

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
        "config": {"workload": wl["desc"], "r": r, "tokens_per_step": T, "microbatch": mb,
                   "projection": "qr-gaussian" if wl["kind"] == "qr" else "rademacher, fixed", "tau": wl["tau"],
                   "weight_norm": "carried from the previous update" if args.carried_norm else "streamed from W"},
        "sketch_accumulate_TFLOPs": round(kern["accumulate"]["TFLOPs_in_step"], 2) if kern else None,
        "sketch_accumulate_frac_bf16_peak": round(kern["accumulate"]["TFLOPs_in_step"] / BF16_PEAK_TFLOPS, 4)
        if kern else None,
        "fused_apply_GBs": round(kern["apply"]["GBs"], 1) if kern else None,
        "fused_apply_frac_hbm_peak": round(kern["apply"]["hbm_frac"], 4) if kern else None,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kern.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(X, D, W, mats, wl):
    """The CPU oracle, untuned, on a bounded sample of the same workload: all 7
    QR projections, one 4096-token microbatch of project + accumulate for all 7
    matrices, and all 7 applies; the step time is extrapolated to 8 microbatches."""
    import numpy as np

    import oracle as orc
    from rank_randomized_gradient_amd import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    r, mb = wl["r"], wl["microbatch"]
    n_mb = wl["tokens"] // mb
    bits = synth.to_numpy_bits
    xs = {name: bits(x[:mb]) for name, x in X.items()}
    ds = [bits(d[:mb]) for d in D]
    ws = [bits(w) for w in W]
    t0 = time.perf_counter()
    ps = [orc.qr_projection(step_seed(0, m), k, r) for m, (_, _, k, _) in enumerate(mats)]
    t1 = time.perf_counter()
    cs = []
    for m, (_, d, k, src) in enumerate(mats):
        c = np.zeros((d, r), np.float32)
        cs.append(orc.accumulate(c, ds[m], orc.project(xs[src], ps[m])))
    t2 = time.perf_counter()
    for m in range(len(mats)):
        orc.apply_update(ws[m], cs[m], ps[m], wl["tau"], step_seed(0, m))
    t3 = time.perf_counter()
    step_s = (t1 - t0) + n_mb * (t2 - t1) + (t3 - t2)
    return {"value": round(wl["tokens"] / step_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"7 QR projections + 1 of {n_mb} microbatches (project+accumulate, 7 matrices) + 7 applies, "
                      f"measured {t3 - t0:.1f}s; step time = projections + {n_mb} x microbatch + applies "
                      f"= {step_s:.1f}s"}


if __name__ == "__main__":
    main()
