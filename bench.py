#!/usr/bin/env python3
"""Benchmark of column-sparse masked attention (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--seed S]

One step is the whole hot path over one batch: the tile pass
(fm_tile_bounds), the forward (fm_attn_fwd) and the backward (fm_attn_bwd),
all through the C ABI, on inputs already resident in device memory.  W untimed
steps; K eager steps with the library's kernel-event hook (per-stage and
per-kernel times); then the step captured once as a HIP graph, W untimed
replays and K timed replays bracketed by torch.cuda.synchronize() (the replay
must reproduce the eager outputs bit for bit, else the eager steps are timed).

The throughput is mask-effective: forward 4*D*nnz and backward 10*D*nnz flops
per (batch, head), nnz being the number of unmasked (query, key) pairs, so
masked work the kernels skip is not credited and masked elements they compute
inside partial tiles are not credited either.

With head_dim 128 the fp8 forward (fm_attn_fwd_fp8, E4M3 inputs) is then
timed on the same workload and reported beside the step ("fp8_forward"; not
part of the step or its throughput).

Printed: one JSON line with the whole-step throughput, the roofline of the
dominant kernel (timed live with HIP events recorded by the library right
around that kernel, on the stream it runs on; medians of the K eager steps)
and the fp64 CPU oracle timed on a bounded sample of the same workload on the
host cores (a reported baseline, not a target).  The headline workload is the
largest one, documents with a 10% bidirectional prefix at B=1, H=8, S=131072,
D=128, seed 4; --config picks another of the five evaluation workloads
(1 causal documents S=1K D=64, 2 sliding window S=8K, 3 share-question S=32K,
5 one context-parallel rank's share).  Unless --only is given, the other
workloads of 8K-128K are timed the same way after it and reported under
"other_workloads" (same fields, no CPU baseline or fp8 line).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mask-effective attention fwd+bwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
# Dense bf16 MFMA peak of MI355X: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0   # HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="the headline workload (default 4, the largest: documents with prefix-LM, S=128K)")
    ap.add_argument("--only", action="store_true",
                    help="time only the headline workload (default: also the other workloads of 8K-128K, "
                         "reported under other_workloads)")
    ap.add_argument("--seed", type=int, default=None, help="default: the config's index")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample (at least one head is always run)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward's line (head_dim 128 only)")
    ap.add_argument("--no-tile-cache", action="store_true",
                    help="run the backward without the tile cache (dQ recomputes S and dP)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="leave out the oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args(argv)


def copy_calibration(nbytes: int) -> int:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}), flush=True)
    return 0


def kernel_source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "column_sparse_masked_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload_tag: str, digest: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 PMC
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration),
    or None when there is none or it was taken on other kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                key, val = ln.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tensors, budget_s):
    """The fp64 oracle (forward + backward) on a bounded sample of the same
    workload: strips of 256 consecutive query rows of head (0, 0), at seeded
    random places, until the time budget is spent (at least one strip).  Each
    strip is the oracle's own unit of work (its rows against every key they
    see).  Mask-effective flops of the sampled rows (14 D times their unmasked
    (i, j) pairs) over the time taken; heads and strips are independent, so
    this is the rate at which the oracle would run the whole workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is one thread per core
        cores = os.cpu_count() or 1
    q, k, v, do = tensors
    up = oracle.upcast_bf16
    b, h = 0, 0
    bh = w.bounds[b, oracle.mask_head(w.bounds, h)]
    qh, kh, vh, doh = up(q[b, h]), up(k[b, h]), up(v[b, h]), up(do[b, h])
    strip = 256
    n_strips = -(-w.Sq // strip)
    order = np.random.default_rng(1000 + w.seed).permutation(n_strips)
    flops, rows_done, strips, dt = 0.0, 0, 0, 0.0
    for s_ in order:
        rows = np.arange(s_ * strip, min(w.Sq, (s_ + 1) * strip))
        t0 = time.perf_counter()
        oh, lse = oracle.head_forward(qh, kh, vh, bh, w.scale, rows)
        oracle.head_backward(qh, kh, vh, doh, bh, w.scale, rows, lse)
        dt += time.perf_counter() - t0
        flops += 14.0 * w.D * float((~oracle.dense_mask(bh, rows)).sum())
        rows_done += rows.size
        strips += 1
        if dt >= budget_s:
            break
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{strips} of {n_strips} strips of 256 query rows ({rows_done} rows) of head (0, 0) of the "
                  f"same workload, forward + backward in float64 numpy, {dt:.1f} s; the rate extrapolates to "
                  f"all {w.B * w.H} (batch, head) pairs, which are independent",
    }


def fp8_forward(w, tensors, att, tb, args, k_fwd_bf16, f_fwd, tag):
    """The fp8 forward (fm_attn_fwd_fp8) on the same workload, inputs encoded
    to E4M3 with per-tensor descales: W untimed calls, then K calls with the
    library's kernel events around the forward kernel.  Mask-effective
    4*D*nnz flops per call, against the fp8 dense matrix-core peak."""
    import numpy as np
    import torch
    from column_sparse_masked_amd import _lib, masks
    from column_sparse_masked_amd.api import to_device_u8
    q8, k8, v8, ds = masks.fp8_inputs(tensors)
    t8 = [to_device_u8(c, tb.device) for c in (q8, k8, v8)]
    o8 = torch.empty((w.B, w.H, w.Sq, w.D), dtype=torch.bfloat16, device=tb.device)
    l8 = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=tb.device)
    for _ in range(args.warmup):
        att.forward_fp8(*t8, ds, tb, o=o8, lse=l8)
    evs = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    for e0, e1 in evs:
        _lib.set_kernel_events(e0, e1)
        att.forward_fp8(*t8, ds, tb, o=o8, lse=l8)
    _lib.set_kernel_events(None, None)
    torch.cuda.synchronize()
    kms = median([a.elapsed_time(b) for a, b in evs])
    achieved = f_fwd / (kms * 1e-3) / 1e12
    return {"kernel": "attn_fwd_fp8_kernel", "dtype": "e4m3", "avg_kernel_ms": round(kms, 4),
            "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": read_traffic("attn_fwd_fp8_kernel", tag, kernel_source_digest(["fwd_fp8.hip", "common.h"])),
            "speedup_vs_bf16_forward_kernel": round(k_fwd_bf16 / kms, 3)}


def tile_pass_bytes(w, nQ, nK):
    """Algorithmic HBM bytes of the tile pass: the bounds read once (16 B per
    key column and mask head), the key-block summaries written and read back
    once, the tile classes, the per-block counts (written, then read by the
    queue kernel), both tile lists and both queues written."""
    bhm = w.B * w.Hm
    return (16 * w.Sk * bhm + 2 * 32 * nK * bhm + nQ * nK * bhm + 2 * 4 * (nQ + nK) * bhm
            + 2 * 2 * nQ * nK * bhm + 4 * w.B * w.H * (nQ + nK))


def median(xs):
    import numpy as np
    return float(np.median(np.asarray(xs, dtype=np.float64)))


def run_workload(cfg, seed, args, dev, with_fp8):
    """Time the whole step (tile pass, forward, backward) on one of the
    evaluation workloads; returns the record and what the CPU baseline needs."""
    import numpy as np
    import torch

    from column_sparse_masked_amd import _lib, masks
    from column_sparse_masked_amd.api import MaskedAttention, to_device_bf16, to_device_bounds

    w = masks.config(cfg, seed)
    print(f"# workload {masks.CONFIG_NAMES[cfg]} seed {w.seed}: drawing inputs", file=sys.stderr, flush=True)
    tensors = w.draw()
    tq, tk, tv, tdo = (to_device_bf16(x, dev) for x in tensors)
    tb = to_device_bounds(w.bounds, dev)
    att = MaskedAttention.for_workload(w, dev)
    o = torch.empty((w.B, w.H, w.Sq, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)

    nnz = w.nnz_total()
    f_fwd, f_bwd = 4.0 * w.D * nnz, 10.0 * w.D * nnz

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()          # creates the HIP event
        return e

    def step(ev=None):
        if ev is not None:
            ev["s0"].record()
        att.tile_bounds(tb)
        if ev is not None:
            ev["s1"].record()
            _lib.set_kernel_events(ev["fk0"], ev["fk1"])
        att.forward(tq, tk, tv, tb, o=o, lse=lse)
        if ev is not None:
            ev["s2"].record()
            _lib.set_kernel_events(ev["bk0"], ev["bk1"], ev["bq0"], ev["bq1"])
        att.backward(tq, tk, tv, o, tdo, lse, tb, dq=dq, dk=dk, dv=dv)
        if ev is not None:
            _lib.set_kernel_events(None, None)
            ev["s3"].record()

    # The backward's workspace holds the tile cache for every non-skipped
    # tile (dQ from the cached dS / scale); it is sized from one tile pass,
    # before any timed work.
    att.tile_bounds(tb)
    cache_bytes = att.reserve_tile_cache() if not args.no_tile_cache else 0
    n_tiles = att.tile_count()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup {args.warmup} steps done ({n_tiles} tiles, workspace {cache_bytes / 2**30:.2f} GiB)",
          file=sys.stderr, flush=True)

    # Eager steps with the library's event hook: per-stage and per-kernel times.
    evs = [{n: new_event() for n in ("s0", "s1", "s2", "s3", "fk0", "fk1", "bk0", "bk1", "bq0", "bq1")}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    ref = [x.clone() for x in (o, lse, dq, dk, dv)]

    # The timed steps: one step captured as a HIP graph and replayed, which
    # removes the launch gaps between the step's kernels.  A replay must
    # reproduce the eager outputs bit for bit, else the eager time is used.
    launch = "hip_graph"
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for x in (o, lse, dq, dk, dv):
            x.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                   for a, b in zip((o, lse, dq, dk, dv), ref)):
            raise RuntimeError("graph replay differs from the eager step")
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
    except Exception as exc:   # graph capture unavailable: time the eager steps instead
        print(f"# graph replay not used ({exc}); timing the eager steps", file=sys.stderr, flush=True)
        launch, wall = "eager", wall_eager
    print(f"# timed {args.steps} steps ({launch}) in {wall:.3f} s; eager {wall_eager:.3f} s",
          file=sys.stderr, flush=True)

    def med_ms(a, b):
        return median([e[a].elapsed_time(e[b]) for e in evs])

    t_tile, t_fwd, t_bwd = med_ms("s0", "s1"), med_ms("s1", "s2"), med_ms("s2", "s3")
    k_fwd, k_bwd, k_dq = med_ms("fk0", "fk1"), med_ms("bk0", "bk1"), med_ms("bq0", "bq1")
    ms_per_step = wall / args.steps * 1e3
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12

    # Per-kernel rooflines: each attention kernel is credited with the
    # mask-effective products that belong to it in the 4 + 10 D nnz
    # accounting: the forward (with its merge of split items) S and PV,
    # 4 D nnz; the dK/dV kernel S, dP, dV, dK, 8 D nnz.  dQ: from the tile
    # cache it is bound by reading the cached tiles, so its roofline is HBM
    # bytes (every cached tile of dS / scale, K once, dQ written); without the
    # cache it recomputes S and dP and is credited with its dQ product only,
    # 2 D nnz (its hardware flops are 6 D nnz).  The dominant kernel is the
    # longest.
    tag = f"cfg{cfg}_seed{w.seed}"
    dq_cached = cache_bytes > 0
    dq_bytes = float(n_tiles) * 128 * 128 * 2 + 2.0 * w.B * w.H * (w.Sk + w.Sq) * w.D
    kernels = {
        "attn_fwd_kernel": ("mfma", 4.0 * w.D * nnz, k_fwd, ["fwd.hip", "common.h"]),
        "attn_bwd_kernel": ("mfma", 8.0 * w.D * nnz, k_bwd, ["bwd.hip", "common.h"]),
        ("attn_bwd_dq_cached_kernel" if dq_cached else "attn_bwd_dq_kernel"):
            ("hbm", dq_bytes, k_dq, ["bwd_dq_cached.hip", "common.h"]) if dq_cached
            else ("mfma", 2.0 * w.D * nnz, k_dq, ["bwd_dq.hip", "common.h"]),
    }

    def roofline(name):
        bound, work, kms, srcs = kernels[name]
        if bound == "mfma":
            achieved, peak, unit, key = work / (kms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", \
                "algorithmic_flops_per_launch"
        else:
            achieved, peak, unit, key = work / (kms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", \
                "algorithmic_bytes_per_launch"
        return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": read_traffic(name, tag, kernel_source_digest(srcs)),
                "avg_kernel_ms": round(kms, 4), "timing": f"median of {args.steps} eager launches, HIP events",
                key: work}

    dom = max(kernels, key=lambda n: kernels[n][2])
    layout = att.buf.layout
    tb_bytes = tile_pass_bytes(w, layout.n_qblocks, layout.n_kblocks)
    rec = {
        "workload": masks.CONFIG_NAMES[cfg],
        "seed": w.seed, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
        "nnz_per_head_mean": nnz / (w.B * w.H),
        "mask_flops_fwd_bwd": f_fwd + f_bwd,
        "step_launch": launch,
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(wall_eager / args.steps * 1e3, 4),
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {"tile_bounds": round(t_tile, 4), "fwd": round(t_fwd, 4), "bwd": round(t_bwd, 4)},
        "kernel_ms": {"fwd": round(k_fwd, 4), "bwd_dkdv": round(k_bwd, 4), "bwd_dq": round(k_dq, 4)},
        "tflops_fwd_kernel": round(f_fwd / (k_fwd * 1e-3) / 1e12, 2),
        "tflops_bwd_kernels_mask_effective": round(f_bwd / ((k_bwd + k_dq) * 1e-3) / 1e12, 2),
        "tflops_without_tile_pass": round((f_fwd + f_bwd) / ((t_fwd + t_bwd) * 1e-3) / 1e12, 2),
        "tile_pass": {"ms": round(t_tile, 4), "algorithmic_bytes": tb_bytes,
                      "GB_per_s": round(tb_bytes / (t_tile * 1e-3) / 1e9, 2), "launches": 2},
        "tile_cache": {"tiles": n_tiles, "workspace_bytes": cache_bytes, "dq_from_cache": dq_cached},
        "roofline": roofline(dom),
        "kernel_rooflines": {n: {k: v for k, v in roofline(n).items()
                                 if k in ("bound", "achieved", "unit", "frac", "avg_kernel_ms")}
                             for n in kernels},
    }
    if with_fp8 and w.D == 128:
        rec["fp8_forward"] = fp8_forward(w, tensors, att, tb, args, k_fwd, f_fwd, tag)
    del tq, tk, tv, tdo, tb, att, o, lse, dq, dk, dv, ref
    torch.cuda.empty_cache()
    return rec, w, tensors


def main(argv=None):
    args = parse_args(argv)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no sharding, no collectives).", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    head, w, tensors = run_workload(args.config, args.seed, args, dev, not args.no_fp8)
    others = {}
    if not args.only:
        for c in (2, 3, 4, 5):
            if c != args.config:
                others[f"config{c}"], _, _ = run_workload(c, None, args, dev, False)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "seed", "B", "H", "Sq", "Sk", "D", "nnz_per_head_mean",
                                         "mask_flops_fwd_bwd", "step_launch")},
    }
    out.update({k: v for k, v in head.items() if k not in out["config"] and k not in ("value", "ms_per_step")})
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        print(f"# oracle sample on the host ({args.cpu_seconds:.0f} s budget)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, tensors, args.cpu_seconds)
    if others:
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
