"""The two ways the backward groups lookups by (table, row) id (kimbodo.com/?p=28372,
"Kimbodo Engineering Perspective": transpose, sort, run-length encoding):

* LSD radix passes followed by a run-length-encoding kernel (TBE_OPTION_SORT = 1);
* for ids of two radix digits, a pass on the high digit followed by a bucket-local sort
  that also run-length encodes (the default where it applies), including ranges longer
  than a workgroup holds in LDS, which are sorted bucket by bucket in chunks.

Both must leave the lookups in the same order (stable on the id), so unique ids, run
lengths, weights and state are bit-identical between them; the default path is also
checked against the CPU reference (runs bit-exact, updates within tolerance)."""
import numpy as np
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import gpu_runs, make_problem, to_device
from test_gpu_parity import _hand_batch, parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _hot_batch(E, B, hot, n_uniform, seed):
    """One table: rows `hot` ({row: hits}) plus n_uniform uniform ids, shuffled into B bags."""
    rng = np.random.default_rng(seed)
    hits = [r for r, k in hot.items() for _ in range(k)] + list(rng.integers(0, E, n_uniform))
    hits = rng.permutation(np.array(hits, np.int64))
    return _hand_batch(1, B, [[list(b) for b in np.array_split(hits, B)]])


# one table of 200 000 rows: 18-bit ids, two 9-bit digits (512 buckets of 512 rows).
# Rows 5 and 600 sit in buckets 0 and 1, row 199 999 in the last nonempty bucket; each of those
# buckets holds more lookups than a workgroup sorts in LDS.
_E_HOT = 200_000
_HOT = {5: 9000, 600: 30000, 199_999: 12000, 77_777: 300}


def _cases():
    return [
        ("workload1", workloads.config(1), None),
        ("workload2", workloads.config(2), None),
        ("hot-buckets", workloads.custom([_E_HOT], [64], "f32", B=512,
                                         optimizer="rowwise_adagrad", key=230),
         [_hot_batch(_E_HOT, 512, _HOT, 100_000, 31)]),
        ("17-bit-mixed", workloads.custom([70_000, 30_000, 1_000], [32, 16, 64], "bf16", B=1500,
                                          lengths=("uniform_int", 0, 40),
                                          index_dist=("zipf", 1.2), pooling="mean", psw=True,
                                          optimizer="rowwise_adagrad", key=231), None),
        ("many-tables", workloads.custom(np.random.default_rng(232).integers(3, 60, 300),
                                         [8] * 300, "f32", B=7, lengths=("uniform_int", 0, 6),
                                         key=232), None),
    ]


CASES = _cases()


def _stages(op):
    return {name for name, _ in op.stage_times()}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bucket_and_lsd_paths_bit_identical(case):
    name, spec, batches = case
    _say(f"[sort paths] {name}")
    a = make_problem(spec, seed=7, batch=None if batches is None else batches[0])
    b = make_problem(spec, seed=7, batch=None if batches is None else batches[0])
    b.op.set_option(tbe.OPTION_SORT, 1)
    a.op.set_option(tbe.OPTION_PROFILE, 1)
    for step in range(2):
        batch = batches[0] if batches is not None else workloads.batch(spec, seed=7, step=step)
        idx, off, psw = to_device(batch)
        G = workloads.grad_output(spec, seed=7, step=step, device="cuda")
        ra, rb = gpu_runs(a, batch.N), gpu_runs(b, batch.N)
        a.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps, ra)
        b.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps, rb)
        torch.cuda.synchronize()
        if step == 0:
            used = _stages(a.op)
            assert "bucket_sort_rle" in used, f"{name}: bucket path not taken ({used})"
            assert "rle_kernel" not in used
        U = int(ra[2].item())
        assert U == int(rb[2].item()) and U > 0
        assert torch.equal(ra[0][:U], rb[0][:U]), f"step {step}: unique ids"
        assert torch.equal(ra[1][:U], rb[1][:U]), f"step {step}: run lengths"
        assert torch.equal(a.W, b.W), f"step {step}: weights"
        if a.state is not None:
            assert torch.equal(a.state, b.state), f"step {step}: state"
        _say(f"  step {step}: identical (U={U})")
    a.op.close()
    b.op.close()


def test_hot_buckets_parity():
    """The chunked path (buckets longer than a workgroup's LDS holds) against the reference."""
    _, spec, batches = CASES[2]
    parity(spec, seed=8, steps=1, batches=batches, row_sample=4000)


def test_17bit_parity_grouped():
    _, spec, _ = CASES[3]
    parity(spec, seed=9, steps=2, grouped=True, bag_sample=2000, row_sample=3000)
