"""Host-side logic of bench.py: its byte model, which is the numerator of every GB/s and
roofline fraction the bench reports, checked against counts made by hand on small
batches; and its refusal of more than one GPU.  No GPU is used."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bytes_of_short_runs_counted_by_hand():
    # two fp32 tables (10 rows of 8 columns, 5 rows of 4), two bags each, sum pooling, SGD:
    # bags t0b0 = [3, 3, 7], t0b1 = [], t1b0 = [1], t1b1 = [1, 4]
    spec = workloads.custom([10, 5], [8, 4], "f32", B=2, key=900)
    batch = workloads.Batch(indices=np.array([3, 3, 7, 1, 1, 4], np.int64),
                            offsets=np.array([0, 3, 3, 4, 6], np.int64), psw=None)
    alg, stats = bench.algorithmic_bytes(spec, batch)
    # forward: per lookup its row (4 * D) and its id (8); per bag its offset (8) and its
    # output row (4 * D)
    fwd = 3 * (4 * 8 + 8) + 3 * (4 * 4 + 8) + 2 * (8 + 4 * 8) + 2 * (8 + 4 * 4)
    assert alg["fwd_gather_pool"] == fwd
    # runs (t0, 3) x 2, (t0, 7) x 1, (t1, 1) x 2, (t1, 4) x 1: all within one lane group
    # (2 lanes at these widths).  Per lookup its sorted value (4) and gradient row (4 * D);
    # per row its id and run bounds (12) and the row read and written (2 * 4 * D)
    seg = (2 * (4 + 32) + 12 + 64) + (1 * (4 + 32) + 12 + 64) \
        + (2 * (4 + 16) + 12 + 32) + (1 * (4 + 16) + 12 + 32)
    assert alg["seg_fused"] == seg
    assert alg["seg_finalize"] == 0
    assert alg["bucket_sort_rle"] == 16 * 6 + 12 * 4
    assert stats == {"N": 6, "U": 4, "long_run_share": 0.0, "max_run": 2}


def test_bytes_of_a_long_run_counted_by_hand():
    # one bf16 table of 4 rows x 8 columns, mean pooling, row-wise Adagrad; one bag holds
    # row 2 six hundred times and row 0 once
    spec = workloads.custom([4], [8], "bf16", B=1, pooling="mean",
                            optimizer="rowwise_adagrad", key=901)
    batch = workloads.Batch(indices=np.array([2] * 600 + [0], np.int64),
                            offsets=np.array([0, 601], np.int64), psw=None)
    alg, stats = bench.algorithmic_bytes(spec, batch)
    assert alg["fwd_gather_pool"] == 601 * (2 * 8 + 8) + (8 + 4 * 8)
    per_look = 4 + 4 * 8 + 8           # sorted value, gradient row, mean's lookup record
    per_row = 12 + 2 * 2 * 8 + 8       # id and bounds, row read and write, Adagrad state
    # row 2: a long run (>= 256) of 3 chunks of 256: every lookup, one fp32 partial written
    # and read back per chunk, then the row; the finish runs inside the segment kernel at
    # this batch size.  Row 0: a short run.
    long_run = 600 * per_look + 3 * 4 * 8 + 3 * 4 * 8 + per_row
    assert alg["seg_fused"] == long_run + (per_look + per_row)
    assert alg["seg_finalize"] == 0
    assert stats["max_run"] == 600 and stats["U"] == 2
    assert abs(stats["long_run_share"] - 600 / 601) < 1e-12
