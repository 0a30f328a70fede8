"""Skew balancing in the forward (TBE_FLAG_SPLIT_BAGS; kimbodo.com/?p=28372, "Kimbodo
Engineering Perspective": load imbalance across lookups is a risk).  Bags of more than 128
lookups are pooled in 128-lookup segments by parallel waves and the segment sums added in
order: the pooled output must match the CPU reference within the forward tolerance, for sum and
mean pooling, with and without per-sample weights, int64 and int32 ids, plain and grouped
calls; the backward is unchanged."""
import numpy as np
import pytest
import torch

import oracle
import table_embedding_bag_amd as tbe
import workloads
from gpu_check import make_problem, to_device
from test_gpu_parity import _hand_batch, parity

pytestmark = pytest.mark.gpu

B = 48
# (table, bag) -> length: one long bag per table, one just over and one exactly at the
# 128-lookup segment length, one a whole number of segments plus one
LONG = {(0, 3): 50000, (0, 10): 129, (0, 11): 128, (1, 20): 9000, (1, 47): 4097}


def _skewed_batch(rows, seed):
    rng = np.random.default_rng(seed)
    bags = []
    for t, E in enumerate(rows):
        tb = []
        for b in range(B):
            L = LONG.get((t, b), int(rng.integers(0, 21)))
            # Zipf-like skew inside the long bags: half the ids from a few hot rows
            ids = rng.integers(0, E, L)
            hot = rng.random(L) < 0.5
            ids[hot] = rng.integers(0, 8, int(hot.sum()))
            tb.append(list(ids))
        bags.append(tb)
    batch = _hand_batch(len(rows), B, bags)
    psw = np.random.default_rng(seed + 1).random(batch.N).astype(np.float32)
    return batch, psw


CASES = [
    workloads.custom([5000, 3000], [128, 64], "f32", B=B, key=260),
    workloads.custom([5000, 3000], [64, 32], "bf16", B=B, pooling="mean", psw=True,
                     optimizer="rowwise_adagrad", key=261),
    workloads.custom([5000, 3000], [48, 24], "f16", B=B, psw=True, key=262),
]


def _batches(spec, seed):
    batch, psw = _skewed_batch(spec.rows, seed)
    return [workloads.Batch(batch.indices, batch.offsets, psw if spec.psw else None)]


@pytest.mark.parametrize("spec", CASES, ids=["f32-sum", "bf16-mean-psw-adagrad", "f16-sum-psw"])
def test_split_bags_parity(spec):
    parity(spec, seed=21, steps=1, batches=_batches(spec, 21), flags=tbe.FLAG_SPLIT_BAGS)


def test_split_bags_grouped_and_int32():
    spec = CASES[1]
    parity(spec, seed=22, steps=1, batches=_batches(spec, 22), flags=tbe.FLAG_SPLIT_BAGS,
           grouped=True)
    parity(spec, seed=23, steps=1, batches=_batches(spec, 23), flags=tbe.FLAG_SPLIT_BAGS,
           index_dtype=torch.int32)


def test_split_bags_launch_and_match_the_reference():
    """The split kernels run for a skewed batch, and its pooled output is within 1e-5 of the
    sum of magnitudes of the fp64 reference (a 50 000-lookup bag: the split sums at most 1024
    terms per lane group before adding the segment sums in order)."""
    spec = CASES[0]
    batch = _batches(spec, 24)[0]
    a = make_problem(spec, seed=24, batch=batch, flags=tbe.FLAG_SPLIT_BAGS)
    a.op.set_option(tbe.OPTION_PROFILE, 1)
    W0 = workloads.storage_numpy(a.W).copy()
    ya = a.op.forward(spec.B, a.idx, a.off, a.psw)
    torch.cuda.synchronize()
    names = {n for n, _ in a.op.stage_times()}
    assert {"fwd_split_segments", "fwd_split_combine"} <= names, names
    y_ref = oracle.forward(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, W0, spec.B,
                           batch.indices, batch.offsets)
    absum = oracle.forward(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, np.abs(W0), spec.B,
                           batch.indices, batch.offsets)
    err = np.abs(ya.cpu().numpy() - y_ref)
    assert (err <= 1e-5 * absum + 1e-30).all(), float((err / (absum + 1e-30)).max())
    a.op.close()
