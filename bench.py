#!/usr/bin/env python3
"""Benchmark of the TBE hot path on one MI355X: forward gather-pool plus the fused
backward (linearize, radix sort, run-length encode, segment reduce, one row-wise
Adagrad / SGD update per touched row), through the library's C ABI.

A step is one forward and one backward update over one batch of the workload:
tbe_forward_group (the pooled lookup, with the backward's linearize step in the
same launch, then the sort and run-length encoding of the batch, which also
queues the longer runs) + tbe_backward_update_grouped (segment reduce and
update: short runs and queued items in one launch, then the long-run finish).
--plain times tbe_forward + tbe_backward_update instead (same results, bit for
bit).  Four seeded batches (and upstream gradients) are generated up front,
resident in HBM, and used in rotation.  The headline workload: T=8 tables of
100,000 x 128 fp32 rows, B=2048 bags per table, bag length uniform in 1..32,
Zipf(1.05) row ids, sum pooling, row-wise Adagrad.

Prints one JSON line:
  value          fwd+bwd lookups per second of the headline workload (lookups of
                 the K timed steps / their wall time)
  roofline       the dominant kernel: algorithmic bytes per launch / its average
                 duration (the kernel's own start/end events, second pass of the
                 same K steps), against the 8 TB/s HBM peak; traffic = HBM bytes
                 per launch from the committed rocprofv3 counter summary when it
                 was taken on the current kernel source, else null
  gates          the two bandwidth gates (plain gather forward; segment reduce +
                 update), each with algorithmic and counter GB/s, with warm caches
                 and with the caches flushed (1 GiB written) before each call
  times          forward, grouping front and segment stage times per step, and
                 forward-only lookups/s
  workloads      the other workloads (mixed widths, hot rows, many small tables):
                 step time, lookups/s, stage times and dominant kernel
  cpu_baseline   the CPU reference's timing build (fp32 accumulators, OpenMP)
                 on the 4 rotated headline batches, median of several rounds, on
                 all host cores and on one
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix-core peak of the MI355X
METRIC = "TBE fwd+bwd lookups/sec and achieved HBM GB/s (% of peak) at 1 MI355X"
FLUSH_BYTES = 1 << 30        # written between calls to empty L2 and the 256 MB MALL
FRONT = ("init_workspace", "linearize_kernel", "radix_count", "radix_scan", "radix_pass",
         "bucket_sort_rle", "rle_count", "rle_kernel")
SEG = ("queue_runs", "table_run_starts", "seg_fused", "seg_finalize")
# calls in each per-kernel and forward-alone pass (at least; more when --steps is larger)
KERNEL_PASS_STEPS = 200
# batches of at most this many lookups have their long runs finished inside seg_fused
FINISH_IN_ITEMS_MAX = 1 << 20
FWD = ("fwd_gather_pool", "fwd_lds_pool", "fwd_linearize", "fwd_histogram", "hist_transpose",
       "fwd_split_segments", "fwd_split_combine")
COUNT_BWD = ("cb_product", "cb_update", "cb_runs")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, help="headline workload 1..5")
    p.add_argument("--extra", default="3,4,5",
                   help="other workloads measured into the same line (comma list, '' for none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU baseline")
    p.add_argument("--forward", choices=("gather", "routed", "histogram"), default="gather",
                   help="gather: the library default (the gather kernel, small tables pooled "
                        "from LDS when a call qualifies); routed: count-matrix forward for the "
                        "tables that qualify; histogram: count-matrix forward for every table "
                        "(all must qualify)")
    p.add_argument("--count-backward", action="store_true",
                   help="the headline workload's handle takes the count-matrix backward "
                        "(every table at most 1024 rows; for its counter collection)")
    p.add_argument("--plain", action="store_true",
                   help="time tbe_forward + tbe_backward_update instead of the grouped pair")
    p.add_argument("--phase", choices=("all", "hot", "flushed"), default="all",
                   help="hot: only the warm-cache passes; flushed: only the flushed-cache pass "
                        "(for counter collection of one kind of call)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device copy of known size (counter calibration)")
    p.add_argument("--histogram-sweep", action="store_true",
                   help="only compare the count-matrix forward with the gather forward over "
                        "table rows E and bag length L (16 bf16 tables, D=64, B=16384, uniform "
                        "ids): one JSON line per (E, L)")
    return p.parse_args()


def histogram_sweep():
    """Crossover of the count-matrix forward against the gather: kernel times (HIP events,
    10 calls after 3 warm-up calls) over E in {64 .. 1024} and L in {4 .. 128}."""
    import torch
    import table_embedding_bag_amd as tbe
    import workloads
    T, D, B = 16, 64, 16384
    for E in (64, 128, 256, 512, 1024):
        for L in (4, 8, 16, 32, 64, 128):
            spec = workloads.custom([E] * T, [D] * T, "bf16", B=B, lengths=("fixed", L), key=900)
            W = workloads.weights(spec, 0, "cuda")
            hb = workloads.batch(spec, 0)
            idx = torch.from_numpy(hb.indices).cuda()
            off = torch.from_numpy(hb.offsets).cuda()
            row = {"E": E, "L": L, "T": T, "D": D, "B": B}
            for mode, flags in (("gather", 0), ("histogram", tbe.FLAG_FORCE_HISTOGRAM)):
                op = tbe.TBE(spec.rows, spec.dims, W, None, pooling="sum", optimizer="sgd",
                             flags=flags)
                for _ in range(3):
                    op.forward(B, idx, off)
                torch.cuda.synchronize()
                op.set_option(tbe.OPTION_PROFILE, 1)
                tbe.tbe_stage_times(op.handle)
                for _ in range(10):
                    op.forward(B, idx, off)
                us = sum(ms for _, ms in tbe.tbe_stage_times(op.handle)) / 10 * 1e3
                row[mode + "_us"] = round(us, 2)
                op.close()
            row["histogram_speedup"] = round(row["gather_us"] / row["histogram_us"], 3)
            print(json.dumps(row), flush=True)
            del W, idx, off
            torch.cuda.empty_cache()


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


def copy_peak():
    """Context for the HBM figures: a plain device copy (torch copy_ of 512 MiB, read plus
    write), timed with events on torch's stream over 10 launches after 3 untimed ones."""
    import torch
    n = 1 << 27
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / 10
    gbps_ = 2 * 4 * n / us / 1e3
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "torch copy_ (512 MiB read + 512 MiB written)", "avg_us": round(us, 1),
            "GBps": round(gbps_, 1), "pct_of_peak": pct(gbps_, HBM_PEAK_GBPS)}


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
                          chunk), in one launch; in batches of at most 2^20 lookups also
                          the long runs' finish (below)
      seg_finalize        per long run: its chunk partials read, the row terms (a launch
                          of its own in batches of more than 2^20 lookups)
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
    if N <= FINISH_IN_ITEMS_MAX:  # the segment kernel finishes the long runs itself
        seg_wg, seg_final = seg_wg + seg_final, 0.0
    front = {"linearize_kernel": float(N * (8 + 8 + rec) + 8 * nbags),
             "radix_pass": float(16 * N), "radix_count": float(4 * N), "rle_count": float(4 * N),
             "rle_kernel": float(4 * N + 16 * U),
             "bucket_sort_rle": float(16 * N + 12 * U),
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
    # the LDS-pooled small tables: the same work per lookup (rows read from LDS), so the
    # same algorithmic bytes as the gather of all tables (a call takes one or the other)
    return {"fwd_gather_pool": fwd, "fwd_lds_pool": fwd,
            "fwd_linearize": fwd + front["linearize_kernel"],
            "fwd_histogram": hist_bytes, "hist_transpose": hist_t,
            "fwd_histogram_flops": hist_flops, "seg_short": seg_short, "seg_wg": seg_wg,
            "seg_fused": seg_short + seg_wg,
            "seg_finalize": seg_final, **front}, {"N": N, "U": U,
                                         "long_run_share": float(cnt[long_].sum() / max(1, cnt.sum())),
                                         "max_run": int(cnt.max()) if cnt.size else 0}


# source file of every kernel (the launch shapes are set next to the kernels)
KERNEL_FILE = {
    "fwd_gather_pool": "forward.hip", "fwd_lds_pool": "forward.hip",
    "fwd_linearize": "forward.hip", "psw_grad": "forward.hip",
    "fwd_split_segments": "forward.hip", "fwd_split_combine": "forward.hip",
    "fwd_histogram": "histogram.hip", "hist_transpose": "histogram.hip",
    "cb_product": "count_backward.hip", "cb_update": "count_backward.hip",
    "cb_runs": "count_backward.hip",
    "init_workspace": "sort.hip", "linearize_kernel": "sort.hip", "radix_pass": "sort.hip",
    "radix_count": "sort.hip", "radix_scan": "sort.hip", "rle_count": "sort.hip",
    "radix_pass_wide": "sort.hip", "bucket_sort_rle": "sort.hip", "rle_kernel": "sort.hip",
    "queue_runs": "segment.hip", "table_run_starts": "segment.hip", "seg_fused": "segment.hip",
    "seg_finalize": "segment.hip",
}


def kernel_source_hash(kernel):
    """Hash of the kernel's source file and of the headers it includes (transitively): a
    counter summary holds for the kernel while this is unchanged."""
    csrc = os.path.join(ROOT, "table_embedding_bag_amd", "csrc")
    names, todo = [], [KERNEL_FILE[kernel]]
    while todo:
        f = todo.pop(0)
        if f in names or not os.path.exists(os.path.join(csrc, f)):
            continue
        names.append(f)
        for line in open(os.path.join(csrc, f)):
            if line.startswith('#include "'):
                todo.append(line.split('"')[1])
    h = hashlib.sha256()
    for f in names:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _summary(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", " ", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def committed_counter(kernel, tag, key="hbm_bytes_per_launch"):
    """A figure from profiles/<kernel>_<tag>_counters.txt (or _mfma.txt for MFMA busy), if
    that summary was taken on the current kernel source; else None."""
    names = {"radix_pass": ("radix_pass", "radix_pass_wide")}.get(kernel, (kernel,))
    suffix = "mfma" if key == "mfma_busy_pct" else "counters"
    for k in names:
        path = os.path.join(ROOT, "profiles", f"{k}_{tag}_{suffix}.txt")
        if not os.path.exists(path):
            continue
        kv = _summary(path)
        if kv.get("kernel_source_sha256_16") != kernel_source_hash(k):
            return None
        try:
            return float(kv[key])
        except (KeyError, ValueError):
            return None
    return None


def gbps(nbytes, us):
    return None if nbytes is None or not us else nbytes / (us * 1e-6) / 1e9


def pct(x, peak):
    return None if x is None else round(100.0 * x / peak, 1)


class Workload:
    """One workload resident on the GPU: tables, state, handle, 4 rotated batches, upstream
    gradients, output and workspace."""

    def __init__(self, n, forward="gather", extra_flags=0):
        import torch
        import table_embedding_bag_amd as tbe
        import workloads
        self.tbe, self.torch = tbe, torch
        self.n = n
        self.spec = spec = workloads.config(n)
        dev = torch.device("cuda:0")
        self.W = workloads.weights(spec, seed=0, device=dev)
        self.state = torch.zeros(spec.sum_rows, dtype=torch.float32, device=dev) \
            if spec.optimizer == "rowwise_adagrad" else None
        flags = {"gather": 0, "routed": tbe.FLAG_HISTOGRAM,
                 "histogram": tbe.FLAG_FORCE_HISTOGRAM}[forward] | extra_flags
        self.forward_mode = forward
        self.op = tbe.TBE(spec.rows, spec.dims, self.W, self.state, pooling=spec.pooling,
                          optimizer=spec.optimizer, flags=flags)
        self.host = [workloads.batch(spec, seed=0, step=s) for s in range(4)]
        self.dev = []
        for hb in self.host:
            idx = torch.from_numpy(hb.indices).to(dev)
            off = torch.from_numpy(hb.offsets).to(dev)
            psw = torch.from_numpy(hb.psw).to(dev) if hb.psw is not None else None
            self.dev.append((idx, off, psw, hb.N))
        self.grads = [workloads.grad_output(spec, seed=0, step=s, device=dev) for s in range(4)]
        self.Y = torch.empty((spec.B, spec.sum_dims), dtype=torch.float32, device=dev)
        self.ws = max((self.op.workspace(spec.B, b[3]) for b in self.dev), key=lambda t: t.numel())
        torch.cuda.synchronize()

    def pair(self, i, plain=False):
        tbe, spec = self.tbe, self.spec
        idx, off, psw, n = self.dev[i % 4]
        G = self.grads[i % 4]
        if plain:
            tbe.tbe_forward(self.op.handle, spec.B, idx, off, psw, self.Y)
            tbe.tbe_backward_update(self.op.handle, spec.B, idx, off, psw, G, spec.lr, spec.eps,
                                    self.ws)
        else:
            tbe.tbe_forward_group(self.op.handle, spec.B, idx, off, psw, self.Y, self.ws)
            tbe.tbe_backward_update_grouped(self.op.handle, spec.B, idx, off, psw, G, spec.lr,
                                            spec.eps, self.ws)
        return n

    def forward(self, i):
        idx, off, psw, n = self.dev[i % 4]
        self.tbe.tbe_forward(self.op.handle, self.spec.B, idx, off, psw, self.Y)
        return n

    def timed(self, fn, start, k):
        """Wall time of k calls of fn(i) (nothing else on the stream), and their lookups."""
        torch = self.torch
        torch.cuda.synchronize()
        lookups, t0 = 0, time.perf_counter()
        for i in range(k):
            lookups += fn(start + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, lookups

    def kernel_times(self, fn, start, k, between=None):
        """{kernel: [ms of each launch]} over k calls of fn(i), from the kernels' own
        start/end events; between(i), if given, runs before each call, untimed."""
        tbe = self.tbe
        self.op.set_option(tbe.OPTION_PROFILE, 1)
        tbe.tbe_stage_times(self.op.handle, capacity=1 << 16)  # drop anything earlier
        out = {}
        for i in range(k):
            if between is not None:
                between(start + i)
            fn(start + i)
            if between is not None:  # read per call, so the untimed work stays outside
                for name, ms in tbe.tbe_stage_times(self.op.handle, capacity=1 << 12):
                    out.setdefault(name, []).append(ms)
        for name, ms in tbe.tbe_stage_times(self.op.handle, capacity=1 << 16):
            out.setdefault(name, []).append(ms)
        self.op.set_option(tbe.OPTION_PROFILE, 0)
        return out

    def close(self):
        self.op.close()
        del self.W, self.state, self.dev, self.grads, self.Y, self.ws
        self.torch.cuda.empty_cache()


def avg_us(times, k, skip_half=False):
    """Average launch time (us) and launches per call, per kernel; skip_half: average over
    the second half of the launches only (the first half of a pass that starts the GPU's
    clock ramp)."""
    def mean(v):
        w = v[len(v) // 2:] if skip_half and len(v) > 1 else v
        return 1e3 * sum(w) / len(w)
    return ({name: mean(v) for name, v in times.items()},
            {name: len(v) / k for name, v in times.items()})


def stage_split(us, per_call):
    """Forward, grouping-front and segment time per step (us) from per-kernel averages."""
    def total(names):
        return sum(us[k] * per_call[k] for k in names if k in us)
    return {"t_fwd_us": round(total(FWD), 2), "t_bwd_front_us": round(total(FRONT), 2),
            "t_bwd_seg_us": round(total(SEG) + total(COUNT_BWD), 2),
            "t_bwd_us": round(total(FRONT) + total(SEG) + total(COUNT_BWD), 2)}


def mean_alg_bytes(wl, gather_tables=None):
    """Algorithmic bytes per launch averaged over the 4 rotated batches, their mean sizes,
    and the sizes of batch 0."""
    import numpy as np
    alg = [algorithmic_bytes(wl.spec, wl.host[i], gather_tables) for i in range(4)]
    return ({k: float(np.mean([a[0][k] for a in alg])) for k in alg[0][0]},
            {k: float(np.mean([a[1][k] for a in alg])) for k in ("N", "U", "long_run_share")},
            alg[0][1])


def measure(wl, args, steps, warmup, headline):
    """The workload's timed step, its kernels, forward-only throughput and (headline)
    the bandwidth gates with warm and flushed caches."""
    torch = wl.torch
    out = {}
    phase = args.phase if headline else "all"
    # host-side statistics first, so that the warm-up steps run right before the timed
    # ones (a GPU left idle between them starts the timed steps at lower clocks)
    routed = [] if wl.forward_mode == "gather" else hist_tables(wl.spec)
    gather = [t for t in range(wl.spec.T) if t not in routed]
    alg, mean_stats, stats0 = mean_alg_bytes(wl, gather)
    out["stats"] = {"lookups_per_step": round(mean_stats["N"]),
                    "unique_rows_per_step": round(mean_stats["U"]),
                    "long_run_share": round(mean_stats["long_run_share"], 3),
                    "batch0": {"lookups": stats0["N"], "unique_rows": stats0["U"],
                               "long_run_share": round(stats0["long_run_share"], 3),
                               "max_run": stats0["max_run"]}}
    if phase in ("all", "hot"):
        # The per-kernel pass and the forward alone come first, over at least
        # KERNEL_PASS_STEPS calls each (finer averages).  They also keep the GPU busy for
        # a few tens of ms before the timed steps: after idling it raises its clocks over
        # about 10 ms of work (workload 2, per 10-step block: 85, 81, 80, ... 77.5 us a
        # step), so a short timed run started cold would measure the ramp.
        ks = max(steps, KERNEL_PASS_STEPS)
        kt = wl.kernel_times(lambda i: wl.pair(i, args.plain), warmup, ks)
        # averages over the pass's second half, past the ramp
        us, per_call = avg_us(kt, ks, skip_half=True)
        out["avg_us"], out["per_call"] = us, per_call
        out["profiled_ms_per_step"] = sum(us[k] * per_call[k] for k in us) / 1e3
        out["times"] = stage_split(us, per_call)
        # forward alone (tbe_forward): its lookups/s and the plain gather kernel
        el_f, look_f = wl.timed(wl.forward, warmup, ks)
        out["times"]["lookups_per_s_fwd"] = round(look_f / el_f, 1)
        out["times"]["t_fwd_call_us"] = round(1e6 * el_f / ks, 2)
        kf = wl.kernel_times(wl.forward, warmup, ks)
        out["fwd_only_us"], _ = avg_us(kf, ks)
    # the warm-up steps, then the timed ones
    for i in range(warmup):
        wl.pair(i, args.plain)
    torch.cuda.synchronize()
    if phase in ("all", "hot"):
        el, lookups = wl.timed(lambda i: wl.pair(i, args.plain), warmup, steps)
        out["elapsed"], out["lookups"] = el, lookups
        print(f"[bench] workload {wl.n}: {steps} steps in {el * 1e3:.2f} ms", file=sys.stderr,
              flush=True)
    if headline and phase in ("all", "flushed"):
        # every call starts with caches emptied by a 1 GiB write: a plain forward, then the
        # grouped pair with a second flush before its backward (its segment kernels then read
        # rows, gradients and state cold)
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")

        def flush(i):
            scratch.fill_(float(i))

        def flushed_step(i):
            spec = wl.spec
            idx, off, psw, n = wl.dev[i % 4]
            wl.forward(i)
            wl.tbe.tbe_forward_group(wl.op.handle, spec.B, idx, off, psw, wl.Y, wl.ws)
            flush(i)
            wl.tbe.tbe_backward_update_grouped(wl.op.handle, spec.B, idx, off, psw,
                                               wl.grads[i % 4], spec.lr, spec.eps, wl.ws)

        kfl = wl.kernel_times(flushed_step, warmup, steps, between=flush)
        out["flushed_us"], _ = avg_us(kfl, steps)
        del scratch
        torch.cuda.empty_cache()
    out["alg"] = alg
    return out


def gate_entry(kernels, alg, us_hot, us_flushed, tag):
    """Algorithmic and counter GB/s of one gated kernel set (summed launch times)."""
    entry = {"kernels": list(kernels), "alg_bytes_per_call": sum(alg[k] for k in kernels)}
    for mode, us, ctag in (("hot", us_hot, tag), ("flushed", us_flushed, f"{tag}_flushed")):
        if us is None or any(k not in us for k in kernels):
            entry[mode] = None
            continue
        t = sum(us[k] for k in kernels)
        cb = [committed_counter(k, ctag) for k in kernels]
        cbytes = None if any(c is None for c in cb) else sum(cb)
        a = gbps(entry["alg_bytes_per_call"], t)
        c = gbps(cbytes, t)
        entry[mode] = {"avg_us": round(t, 2), "alg_GBps": round(a, 1), "pct_peak_alg": pct(a, HBM_PEAK_GBPS),
                       "counter_bytes_per_call": cbytes,
                       "counter_GBps": None if c is None else round(c, 1),
                       "pct_peak_counter": pct(c, HBM_PEAK_GBPS)}
    return entry


def kernel_table(m):
    us, per_call, alg = m.get("avg_us", {}), m.get("per_call", {}), m["alg"]
    out = {}
    for k, t in us.items():
        e = {"avg_us": round(t, 2), "launches_per_step": round(per_call[k], 2)}
        if k in alg:
            e["alg_bytes"] = alg[k]
            e["alg_GBps"] = round(gbps(alg[k], t), 1)
            e["pct_of_peak_alg"] = pct(gbps(alg[k], t), HBM_PEAK_GBPS)
        out[k] = e
    return out


def dominant_roofline(m, tag):
    us, per_call, alg = m["avg_us"], m["per_call"], m["alg"]
    dom = max(us, key=lambda k: us[k] * per_call[k])
    if dom == "fwd_histogram" and alg.get("fwd_histogram_flops"):
        tf = alg["fwd_histogram_flops"] / (us[dom] * 1e-6) / 1e12
        return {"bound": "mfma", "kernel": dom, "achieved": round(tf, 1),
                "peak": MFMA16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA16_PEAK_TFLOPS, 4),
                "traffic": committed_counter(dom, tag),
                "alg_flops_per_launch": alg["fwd_histogram_flops"],
                "avg_launch_us": round(us[dom], 2)}
    if dom in alg:
        a = gbps(alg[dom], us[dom])
        return {"bound": "hbm", "kernel": dom, "achieved": round(a, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(a / HBM_PEAK_GBPS, 4),
                "traffic": committed_counter(dom, tag), "alg_bytes_per_launch": alg[dom],
                "avg_launch_us": round(us[dom], 2)}
    return {"bound": "hbm", "kernel": dom, "achieved": None, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": None, "traffic": None, "avg_launch_us": round(us[dom], 2)}


def histogram_forward(args, steps, warmup):
    """Forward-only figures of the count-matrix (MFMA) forward on the many-small-tables
    workload: every table routed to it."""
    wl = Workload(5, forward="histogram")
    try:
        for i in range(warmup):
            wl.forward(i)
        el, look = wl.timed(wl.forward, warmup, steps)
        kt = wl.kernel_times(wl.forward, warmup, steps)
        us, _ = avg_us(kt, steps)
        alg, _, _ = mean_alg_bytes(wl, [])
        t = us.get("fwd_histogram")
        tf = alg["fwd_histogram_flops"] / (t * 1e-6) / 1e12 if t else None
        return {"lookups_per_s_fwd": round(look / el, 1), "t_fwd_call_us": round(1e6 * el / steps, 2),
                "kernel_avg_us": {k: round(v, 2) for k, v in us.items()},
                "TFLOPs": None if tf is None else round(tf, 1),
                "pct_of_mfma_peak": None if tf is None else round(100 * tf / MFMA16_PEAK_TFLOPS, 1),
                "alg_GBps": round(gbps(alg["fwd_histogram"], t), 1) if t else None,
                "mfma_busy_pct": committed_counter("fwd_histogram", "workload5", "mfma_busy_pct")}
    finally:
        wl.close()


def count_backward(args, steps, warmup):
    """The many-small-tables workload with the count-matrix backward (no sort): step time,
    backward time and the product's rate against the dense bf16 MFMA peak."""
    import table_embedding_bag_amd as tbe
    wl = Workload(5, extra_flags=tbe.FLAG_COUNT_BACKWARD)
    try:
        for i in range(warmup):
            wl.pair(i)
        el, look = wl.timed(wl.pair, warmup, steps)
        kt = wl.kernel_times(wl.pair, warmup, steps)
        us, per_call = avg_us(kt, steps)
        spec = wl.spec
        # three bf16 parts of G times the count matrix: 3 x 2 B E_t D_t per table
        flops = float(sum(3 * 2 * spec.B * e * d for e, d in zip(spec.rows, spec.dims)))
        t = us.get("cb_product")
        tf = flops / (t * 1e-6) / 1e12 if t else None
        bwd = sum(us[k] * per_call[k] for k in ("cb_product", "cb_update", "cb_runs") if k in us)
        return {"ms_per_step": round(1e3 * el / steps, 4), "lookups_per_s": round(look / el, 1),
                "t_bwd_us": round(bwd, 2),
                "kernel_avg_us": {k: round(v, 2) for k, v in us.items()},
                "product_alg_flops": flops,
                "product_TFLOPs": None if tf is None else round(tf, 1),
                "product_pct_of_mfma_peak": None if tf is None else round(100 * tf / MFMA16_PEAK_TFLOPS, 1),
                "mfma_busy_pct": committed_counter("cb_product", "workload5", "mfma_busy_pct")}
    finally:
        wl.close()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, W_host, budget_s):
    """The CPU reference as it stands, in its timing build (fp32 accumulators, gcc -O3
    -march=native -fopenmp, compiled here for this host): forward and backward_update on
    each of the 4 rotated batches, rounds repeated (at least 3) within the budget, median
    per call; then one round on a single thread."""
    import numpy as np
    import oracle
    import workloads
    spec = wl.spec
    path = os.path.join(tempfile.mkdtemp(prefix="tbe_oracle_"), "libtbe_oracle_f32.so")
    lib = oracle.load_timed(oracle.build_timed(path))
    dt = workloads.oracle_dtype(spec.dtype)
    pool = oracle.POOL_MEAN if spec.pooling == "mean" else oracle.POOL_SUM
    opt = oracle.OPT_ROWWISE_ADAGRAD if spec.optimizer == "rowwise_adagrad" else oracle.OPT_SGD
    grads = [g.cpu().numpy() for g in wl.grads]
    W = W_host.copy()
    st = np.zeros(spec.sum_rows, np.float32)
    lr, eps = float(np.float32(spec.lr)), float(np.float32(spec.eps))

    def one_round(times):
        for b, G in zip(wl.host, grads):
            t0 = time.perf_counter()
            oracle.forward(spec.rows, spec.dims, dt, pool, W, spec.B, b.indices, b.offsets,
                           b.psw, lib=lib)
            t1 = time.perf_counter()
            oracle.backward_update(spec.rows, spec.dims, dt, pool, opt, W, st, spec.B, b.indices,
                                   b.offsets, b.psw, G, lr, eps, lib=lib)
            t2 = time.perf_counter()
            times.append((t1 - t0, t2 - t1, b.N))

    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads, lib)
    many, rounds, t_start = [], 0, time.perf_counter()
    while rounds < 3 or (time.perf_counter() - t_start < budget_s and rounds < 20):
        one_round(many)
        rounds += 1
    oracle.set_threads(1, lib)
    single = []
    one_round(single)
    oracle.set_threads(threads, lib)

    def summary(times):
        f = statistics.median(t[0] for t in times)
        b = statistics.median(t[1] for t in times)
        n = statistics.mean(t[2] for t in times)
        return f, b, n

    f, b, n = summary(many)
    f1, b1, _ = summary(single)
    return {"value": round(n / (f + b), 1), "unit": "lookups/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rounds} rounds over the 4 rotated batches ({round(n)} lookups each): "
                      f"forward + backward_update, median per call, fp32 accumulators, "
                      f"{threads} threads; then 1 round on one thread",
            "fwd_ms": round(1e3 * f, 2), "bwd_update_ms": round(1e3 * b, 2),
            "lookups_per_s_fwd": round(n / f, 1),
            "value_1thread": round(n / (f1 + b1), 1), "fwd_ms_1thread": round(1e3 * f1, 2),
            "bwd_update_ms_1thread": round(1e3 * b1, 2), "cpu_model": cpu_model(),
            "build": "oracle/tbe_oracle.c, -DORACLE_ACC=float -O3 -march=native -fopenmp"}


def workload_line(wl, m, steps):
    """Summary of one of the other workloads for the JSON line."""
    out = {"workload": wl.spec.name, **m["stats"]}
    if "elapsed" in m:
        out["ms_per_step"] = round(1e3 * m["elapsed"] / steps, 4)
        out["lookups_per_s"] = round(m["lookups"] / m["elapsed"], 1)
        out.update(m["times"])
        r = dominant_roofline(m, f"workload{wl.n}")
        r.pop("peak", None)
        out["dominant"] = r
        out["kernels"] = kernel_table(m)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path (tables are not sharded across GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.histogram_sweep:
        histogram_sweep()
        return

    import torch
    import workloads

    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    import table_embedding_bag_amd as tbe
    wl = Workload(args.workload, args.forward,
                  tbe.FLAG_COUNT_BACKWARD if args.count_backward else 0)
    W_host = workloads.storage_numpy(wl.W).copy() \
        if not args.no_cpu_baseline and args.phase == "all" else None
    print(f"[bench] workload {args.workload} ready in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    m = measure(wl, args, args.steps, args.warmup, headline=True)
    tag = f"workload{args.workload}"
    if args.phase != "all":
        print(json.dumps({"phase": args.phase, "workload": args.workload,
                          "kernel_avg_us": {k: round(v, 2) for k, v in
                                            m.get("avg_us", m.get("flushed_us", {})).items()}}))
        wl.close()
        return

    gates = {
        "forward_gather_pool": gate_entry(("fwd_gather_pool",), m["alg"], m["fwd_only_us"],
                                          m.get("flushed_us"), tag),
        "segment_reduce_update": gate_entry(
            tuple(k for k in ("seg_fused", "seg_finalize") if k in m["avg_us"]), m["alg"],
            m["avg_us"], m.get("flushed_us"), tag),
        "threshold_pct": 60,
        "note": "alg = the method's own bytes (one row read per lookup); counter = "
                "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch (committed summaries, same "
                "source), both over the live launch time; hot = caches warm, flushed = "
                "1 GiB written before each call",
    }
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU reference", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, W_host, args.cpu_seconds)
    roofline = dominant_roofline(m, tag)
    spec = wl.spec
    value = m["lookups"] / m["elapsed"]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * m["elapsed"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded generator, 4 rotated batches resident in HBM)",
        "config": {"workload": spec.name, "tables": spec.T, "bags_per_table": spec.B,
                   "forward": args.forward,
                   "calls": "tbe_forward + tbe_backward_update" if args.plain
                            else "tbe_forward_group + tbe_backward_update_grouped",
                   **m["stats"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gates": gates,
        "copy_kernel": copy_peak(),
        "times": m["times"],
        "kernels": kernel_table(m),
        "profiled_ms_per_step": round(m["profiled_ms_per_step"], 4),
    }
    steps_x = min(args.steps, 20)
    wl.close()
    del wl
    others = {}
    for n in [int(x) for x in args.extra.split(",") if x.strip()]:
        if n == args.workload:
            continue
        try:
            t0 = time.perf_counter()
            w = Workload(n)
            print(f"[bench] workload {n} ready in {time.perf_counter() - t0:.1f}s",
                  file=sys.stderr, flush=True)
            others[f"workload{n}"] = workload_line(w, measure(w, args, steps_x, 3, False), steps_x)
            w.close()
            if n == 5:
                others["workload5"]["count_matrix_forward"] = histogram_forward(args, steps_x, 3)
                others["workload5"]["count_matrix_backward"] = count_backward(args, steps_x, 3)
        except Exception as e:  # report, keep the headline line
            others[f"workload{n}"] = {"error": f"{type(e).__name__}: {e}"}
    out["workloads"] = others
    print(json.dumps(out))


if __name__ == "__main__":
    main()
