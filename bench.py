#!/usr/bin/env python3
"""Benchmark of the TBE hot path on one MI355X: forward gather-pool plus the fused
backward (linearize, radix sort, run-length encode, segment reduce, one row-wise
Adagrad / SGD update per touched row), through the library's C ABI.

A step is one forward and one backward update over one batch of the workload:
tbe_forward_group (the pooled lookup, with the backward's linearize step in the
same launch, then the sort and run-length encoding of the batch, which also
queues the longer runs) + tbe_backward_update_grouped (segment reduce and
update: short runs and queued items in one launch, then the long-run finish).  --plain times
tbe_forward + tbe_backward_update instead (same results, bit for bit).  Four
seeded batches (and
upstream gradients) are generated up front, resident in HBM, and used in
rotation.  Default workload: T=8 tables of 100,000 x 128
fp32 rows, B=2048 bags per table, bag length uniform in 1..32, Zipf(1.05) row
ids, sum pooling, row-wise Adagrad.

Prints one JSON line:
  value        fwd+bwd lookups per second (lookups of the K timed steps / time)
  roofline     the dominant kernel: algorithmic bytes per launch / its average
               duration (the kernel's own start/end events, second pass of the
               same K steps), against the 8 TB/s HBM peak; traffic from the
               committed rocprofv3 counter summary when it matches the current
               kernel source, else null
  cpu_baseline the CPU reference (fp64, OpenMP) timed on a bounded sample of
               the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix-core peak of the MI355X
METRIC = "TBE fwd+bwd lookups/sec and achieved HBM GB/s (% of peak) at 1 MI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, help="benchmark workload 1..5")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU baseline")
    p.add_argument("--forward", choices=("gather", "routed", "histogram"), default="gather",
                   help="gather: the gather forward (the library default); routed: count-matrix "
                        "forward for the tables that qualify; histogram: count-matrix forward "
                        "for every table (all must qualify)")
    p.add_argument("--plain", action="store_true",
                   help="time tbe_forward + tbe_backward_update instead of the grouped pair "
                        "tbe_forward_group + tbe_backward_update_grouped (the backward's "
                        "grouping done with the forward)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device copy of known size (counter calibration)")
    return p.parse_args()


def copy_probe():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "launches": 5}))


def row_stats(spec, batch):
    """Runs of equal (table, row) ids: their lengths, from the batch itself."""
    import numpy as np
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    bag = np.repeat(np.arange(spec.T * spec.B), np.diff(batch.offsets))
    lin = roff[bag // spec.B] + batch.indices
    uniq, cnt = np.unique(lin, return_counts=True)
    tab = np.searchsorted(roff, uniq, side="right") - 1
    return uniq, cnt, tab


def group_lanes(spec):
    """Lanes per gradient row in the segment kernels (longest run a lane group takes alone)."""
    ve = 4 if all(d % 4 == 0 for d in spec.dims) else 1
    c = -(-max(spec.dims) // ve)
    return min(64, 1 << (c - 1).bit_length())


def hist_tables(spec):
    """Tables the count-matrix forward takes when routed: 16-bit storage, at most 1024 rows,
    dims a multiple of 16 up to 256."""
    return [t for t in range(spec.T) if spec.dtype != "f32" and spec.rows[t] <= 1024
            and spec.dims[t] <= 256 and spec.dims[t] % 16 == 0]


def algorithmic_bytes(spec, batch, gather_tables=None, long_threshold=256, chunk=256):
    """Bytes the method itself must move, per kernel (one launch each), for one batch.

    forward (per lookup)  row read D*s + id 8 (+ weight 4); (per bag) offset 8 + output 4*D
                          (gather kernel: the tables in gather_tables, default all)
    fwd_linearize         the gather forward's bytes plus the linearize step's
    segment (per lookup)  sorted value 4 + gradient row 4*D (+ record 8 with weights / mean)
            (per row)     id + run bounds 12 + row read and write 2*D*s (+ state read/write 8)
      seg_fused           short runs (at most Gs lookups, one lane group each) and the
                          queued items: longer runs below the long-run threshold, and the
                          lookups of long runs (+ one 4*D partial write per 256-lookup
                          chunk), in one launch
      seg_finalize        per long run: its chunk partials read, the row terms
    grouping front: linearize, radix passes (key+value read and scatter 16 per lookup),
    bucket_sort_rle (key+value read and final write 16 per lookup; unique id, start and
    first value 12 per run), rle_kernel (keys 4 per lookup; per run 12 written, first
    value read 4), queue_runs (run bounds 8 per run)
    """
    import numpy as np
    s = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    dims = np.array(spec.dims, np.int64)
    lens = np.diff(batch.offsets)
    bag_t = np.repeat(np.arange(spec.T), spec.B)
    look_D = np.repeat(dims[bag_t], lens)
    psw = 4 if spec.psw else 0
    gt = np.ones(spec.T, bool) if gather_tables is None else np.isin(np.arange(spec.T), gather_tables)
    look_g = np.repeat(gt[bag_t], lens)
    fwd = float((look_D * s + 8 + psw)[look_g].sum() + (8 + 4 * dims[bag_t])[gt[bag_t]].sum())
    _, cnt, tab = row_stats(spec, batch)
    D = dims[tab]
    rec = 8 if (spec.psw or spec.pooling == "mean") else 0
    state = 8 if spec.optimizer == "rowwise_adagrad" else 0
    gs = group_lanes(spec)
    per_look = 4 + 4 * D + rec
    per_row = 12 + 2 * D * s + state
    short = cnt <= gs
    long_ = cnt >= long_threshold
    medium = ~short & ~long_
    nch = -(-cnt // chunk)
    seg_short = float((cnt[short] * per_look[short] + per_row[short]).sum())
    seg_wg = float((cnt[medium] * per_look[medium] + per_row[medium]).sum()
                   + (cnt[long_] * per_look[long_] + nch[long_] * 4 * D[long_]).sum())
    seg_final = float((nch[long_] * 4 * D[long_] + per_row[long_]).sum())
    N, U, nbags = int(lens.sum()), int(cnt.size), spec.T * spec.B
    # grouping front: workspace clear (a few KB), linearize (ids 8 + offsets, key/value
    # writes 8, record 8), per radix pass the key+value read and scatter 16 per lookup,
    # run-length encoding keys read 4 + unique id/start writes 8 per run
    front = {"linearize_kernel": float(N * (8 + 8 + rec) + 8 * nbags),
             "radix_pass": float(16 * N), "rle_kernel": float(4 * N + 16 * U),
             "bucket_sort_rle": float(16 * N + 12 * U),
             # run bounds read 8 per run (the few queued runs' entries are not counted)
             "queue_runs": float(8 * U)}
    # count-matrix forward (tables that qualify): ids 8 + per bag offset 8 + output 4*D, one
    # read of each table; the dense product does 2*B*E_t*D_t flops per table.  The W^T
    # staging kernel reads each table and writes its transposed copy.
    s16 = 2
    hist = hist_tables(spec)
    hist_n = sum(int(lens[t * spec.B:(t + 1) * spec.B].sum()) for t in hist)
    hist_bytes = float(8 * hist_n + sum(8 * spec.B + 4 * spec.B * spec.dims[t]
                                        + s16 * spec.rows[t] * spec.dims[t] for t in hist))
    hist_flops = float(sum(2 * spec.B * spec.rows[t] * spec.dims[t] for t in hist))
    hist_t = float(sum(2 * s16 * spec.rows[t] * spec.dims[t] for t in hist))
    return {"fwd_gather_pool": fwd, "fwd_linearize": fwd + front["linearize_kernel"],
            "fwd_histogram": hist_bytes, "hist_transpose": hist_t,
            "fwd_histogram_flops": hist_flops, "seg_short": seg_short, "seg_wg": seg_wg,
            "seg_fused": seg_short + seg_wg,
            "seg_finalize": seg_final, **front}, {"N": int(lens.sum()), "U": int(cnt.size),
                                         "long_run_share": float(cnt[long_].sum() / max(1, cnt.sum())),
                                         "max_run": int(cnt.max()) if cnt.size else 0}


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "table_embedding_bag_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload_tag):
    """HBM bytes per launch from profiles/<kernel>_<workload>_counters.txt, if it was
    taken on the current kernel source (else None)."""
    # a radix pass is timed as one stage whichever kernel variant ran it
    names = {"radix_pass": ("radix_pass", "radix_pass_wide")}.get(kernel, (kernel,))
    paths = [os.path.join(ROOT, "profiles", f"{k}_{workload_tag}_counters.txt") for k in names]
    paths = [p for p in paths if os.path.exists(p)]
    if not paths:
        return None
    path = paths[0]
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(spec, batch, W_host, grad_host, budget_s):
    """The CPU reference as it stands (fp64, OpenMP over bags and rows): forward +
    backward_update on the full first batch, repeated while within the budget."""
    import numpy as np
    import oracle
    import workloads
    dt = workloads.oracle_dtype(spec.dtype)
    pool = oracle.POOL_MEAN if spec.pooling == "mean" else oracle.POOL_SUM
    opt = oracle.OPT_ROWWISE_ADAGRAD if spec.optimizer == "rowwise_adagrad" else oracle.OPT_SGD
    W = W_host.copy()
    st = np.zeros(spec.sum_rows, np.float32)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(spec.rows, spec.dims, dt, pool, W, spec.B, batch.indices, batch.offsets,
                       batch.psw)
        oracle.backward_update(spec.rows, spec.dims, dt, pool, opt, W, st, spec.B, batch.indices,
                               batch.offsets, batch.psw, grad_host, float(np.float32(spec.lr)),
                               float(np.float32(spec.eps)))
        reps += 1
        el = time.perf_counter() - t0
        if el > budget_s or reps >= 20:
            break
    return {"value": reps * batch.N / el, "unit": "lookups/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"{reps} x one full batch ({batch.N} lookups): forward + backward_update, "
                      f"fp64, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import numpy as np
    import torch

    import table_embedding_bag_amd as tbe
    import workloads

    torch.cuda.set_device(0)
    spec = workloads.config(args.workload)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    W = workloads.weights(spec, seed=0, device=dev)
    W_host = workloads.storage_numpy(W).copy() if not args.no_cpu_baseline else None
    state = torch.zeros(spec.sum_rows, dtype=torch.float32, device=dev) \
        if spec.optimizer == "rowwise_adagrad" else None
    fwd_flags = {"gather": 0, "routed": tbe.FLAG_HISTOGRAM,
                 "histogram": tbe.FLAG_FORCE_HISTOGRAM}[args.forward]
    op = tbe.TBE(spec.rows, spec.dims, W, state, pooling=spec.pooling, optimizer=spec.optimizer,
                 flags=fwd_flags)
    nrot = 4
    host_batches = [workloads.batch(spec, seed=0, step=s) for s in range(nrot)]
    batches = []
    for hb in host_batches:
        idx = torch.from_numpy(hb.indices).to(dev)
        off = torch.from_numpy(hb.offsets).to(dev)
        psw = torch.from_numpy(hb.psw).to(dev) if hb.psw is not None else None
        batches.append((idx, off, psw, hb.N))
    grads = [workloads.grad_output(spec, seed=0, step=s, device=dev) for s in range(nrot)]
    Y = torch.empty((spec.B, spec.sum_dims), dtype=torch.float32, device=dev)
    ws = max((op.workspace(spec.B, n) for (_, _, _, n) in batches), key=lambda t: t.numel())
    torch.cuda.synchronize()
    print(f"[bench] workload {args.workload} ready in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)

    def step(i):
        idx, off, psw, n = batches[i % nrot]
        if args.plain:
            tbe.tbe_forward(op.handle, spec.B, idx, off, psw, Y)
            tbe.tbe_backward_update(op.handle, spec.B, idx, off, psw, grads[i % nrot], spec.lr,
                                    spec.eps, ws)
        else:
            tbe.tbe_forward_group(op.handle, spec.B, idx, off, psw, Y, ws)
            tbe.tbe_backward_update_grouped(op.handle, spec.B, idx, off, psw, grads[i % nrot],
                                            spec.lr, spec.eps, ws)
        return n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, nothing else on the stream
    lookups = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        lookups += step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {elapsed * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # second pass over the same K steps with HIP events after every kernel
    op.set_option(tbe.OPTION_PROFILE, 1)
    tbe.tbe_stage_times(op.handle, capacity=1 << 16)  # drop anything earlier
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    stages = tbe.tbe_stage_times(op.handle, capacity=1 << 16)
    op.set_option(tbe.OPTION_PROFILE, 0)
    per_kernel = {}
    for name, ms in stages:
        tot, cnt = per_kernel.get(name, (0.0, 0))
        per_kernel[name] = (tot + ms, cnt + 1)
    avg_us = {k: 1e3 * t / c for k, (t, c) in per_kernel.items()}
    steps_per_launch = {k: c / args.steps for k, (t, c) in per_kernel.items()}

    # algorithmic bytes per launch (averaged over the rotated batches used)
    routed = [] if args.forward == "gather" else hist_tables(spec)
    gather = [t for t in range(spec.T) if t not in routed]
    alg = [algorithmic_bytes(spec, host_batches[(args.warmup + i) % nrot], gather)
           for i in range(nrot)]
    alg_bytes = {k: float(np.mean([a[0][k] for a in alg])) for k in alg[0][0]}
    stats = alg[0][1]
    kernels = {}
    for k, b in alg_bytes.items():
        if k == "fwd_histogram" and k in avg_us:
            fl = alg_bytes["fwd_histogram_flops"]
            kernels[k] = {"avg_us": round(avg_us[k], 2), "alg_bytes": b,
                          "alg_GBps": round(b / (avg_us[k] * 1e-6) / 1e9, 1),
                          "pct_of_peak": round(100 * b / (avg_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
                          "alg_flops": fl, "TFLOPs": round(fl / (avg_us[k] * 1e-6) / 1e12, 1),
                          "pct_of_mfma_peak": round(100 * fl / (avg_us[k] * 1e-6) / 1e12
                                                    / MFMA16_PEAK_TFLOPS, 1)}
        elif k in avg_us:
            kernels[k] = {"avg_us": round(avg_us[k], 2), "alg_bytes": b,
                          "alg_GBps": round(b / (avg_us[k] * 1e-6) / 1e9, 1),
                          "pct_of_peak": round(100 * b / (avg_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}
    # the whole segment reduce + update (all of its kernels, one launch each per step)
    seg_names = [k for k in ("seg_short", "seg_wg", "seg_fused", "seg_finalize") if k in avg_us]
    if seg_names:
        sb, su = sum(alg_bytes[k] for k in seg_names), sum(avg_us[k] for k in seg_names)
        kernels["segment_reduce_update"] = {
            "avg_us": round(su, 2), "alg_bytes": sb, "alg_GBps": round(sb / (su * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100 * sb / (su * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}
    dominant = max(avg_us, key=lambda k: avg_us[k] * steps_per_launch[k])
    workload_tag = f"workload{args.workload}"
    if dominant == "fwd_histogram" and alg_bytes.get("fwd_histogram_flops"):
        tflops = alg_bytes["fwd_histogram_flops"] / (avg_us[dominant] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(tflops, 1),
                    "peak": MFMA16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA16_PEAK_TFLOPS, 4),
                    "traffic": committed_traffic(dominant, f"workload{args.workload}"),
                    "alg_flops_per_launch": alg_bytes["fwd_histogram_flops"],
                    "avg_launch_us": round(avg_us[dominant], 2)}
    elif dominant in alg_bytes:
        achieved = alg_bytes[dominant] / (avg_us[dominant] * 1e-6) / 1e9
        traffic = committed_traffic(dominant, workload_tag)
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic, "alg_bytes_per_launch": alg_bytes[dominant],
                    "avg_launch_us": round(avg_us[dominant], 2)}
    else:
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": None, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": None, "traffic": None,
                    "avg_launch_us": round(avg_us[dominant], 2)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU reference", file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, host_batches[0], W_host, grads[0].cpu().numpy(), args.cpu_seconds)

    value = lookups / elapsed
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16 storage, f32 accumulate",
                  "bf16": "bf16 storage, f32 accumulate"}[spec.dtype],
        "data": "synthetic (seeded generator, 4 rotated batches resident in HBM)",
        "config": {"workload": spec.name, "tables": spec.T, "bags_per_table": spec.B,
                   "forward": args.forward,
                   "calls": "tbe_forward + tbe_backward_update" if args.plain
                            else "tbe_forward_group + tbe_backward_update_grouped",
                   "lookups_per_step": stats["N"], "unique_rows_batch0": stats["U"],
                   "long_run_share_batch0": round(stats["long_run_share"], 3),
                   "max_run_batch0": stats["max_run"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernel_avg_us": {k: round(v, 2) for k, v in avg_us.items()},
        "launches_per_step": {k: round(v, 2) for k, v in steps_per_launch.items()},
        "profiled_ms_per_step": round(sum(ms for _, ms in stages) / args.steps, 4),
    }
    print(json.dumps(out))
    op.close()


if __name__ == "__main__":
    main()
