"""The two ways the backward groups lookups by (table, row) id (kimbodo.com/?p=28372,
"Kimbodo Engineering Perspective": transpose, sort, run-length encoding):

* LSD radix passes followed by a run-length-encoding kernel (TBE_OPTION_SORT = 1);
* for ids of two radix digits, a pass on the high digit followed by a bucket-local sort
  that also run-length encodes (the default where it applies), including ranges longer
  than a workgroup holds in LDS, which are sorted bucket by bucket in chunks.

Both must leave the lookups in the same order (stable on the id), so unique ids, run
lengths, weights and state are bit-identical between them; the default path is also
checked against the CPU reference (runs bit-exact, updates within tolerance).

When a batch has at most 256 linearize tiles (128 bags each), the pass on the high digit is
done by the linearize step itself (in the stand-alone linearize kernel, or in the launch that
also pools the forward when the grouping runs with the forward); with more tiles it is a
radix pass of its own.  Cases on both sides of that limit, plain and grouped, check that
every variant leaves the same order."""
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
        ("tiny-2x1000", workloads.config(1), None),
        ("8x100k-zipf", workloads.config(2), None),
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
        # 2 x 16384 bags: 256 linearize tiles (the linearize step scatters)
        ("256-tiles", workloads.custom([100_000, 50_000], [32, 32], "f32", B=16384,
                                       lengths=("uniform_int", 0, 6), index_dist=("zipf", 1.1),
                                       optimizer="rowwise_adagrad", key=233), None),
        # 3 x 10923 bags: 257 tiles (a radix pass of its own)
        ("257-tiles", workloads.custom([100_000, 50_000, 3_000], [32, 16, 32], "bf16", B=10923,
                                       lengths=("uniform_int", 0, 6), index_dist=("zipf", 1.1),
                                       pooling="mean", psw=True, key=234), None),
        # one tile of 100 bags
        ("one-tile", workloads.custom([5_000], [64], "f32", B=100, lengths=("uniform_int", 0, 40),
                                      index_dist=("zipf", 1.3), optimizer="rowwise_adagrad",
                                      key=235), None),
    ]


CASES = _cases()


def _stages(op):
    return {name for name, _ in op.stage_times()}


def _linearize_tiles(spec):
    return (spec.T * spec.B + 127) // 128


def _update(pb, spec, idx, off, psw, G, runs, grouped):
    if grouped:
        pb.op.forward_group(spec.B, idx, off, psw)
        pb.op.backward_update_grouped(spec.B, idx, off, psw, G, spec.lr, spec.eps, runs)
    else:
        pb.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps, runs)


@pytest.mark.parametrize("grouped", [False, True], ids=["plain", "grouped"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bucket_and_lsd_paths_bit_identical(case, grouped):
    name, spec, batches = case
    _say(f"[sort paths] {name} grouped={grouped}")
    idt = torch.int32 if name in ("256-tiles", "one-tile") else torch.int64
    a = make_problem(spec, seed=7, batch=None if batches is None else batches[0], index_dtype=idt)
    b = make_problem(spec, seed=7, batch=None if batches is None else batches[0], index_dtype=idt)
    b.op.set_option(tbe.OPTION_SORT, 1)
    a.op.set_option(tbe.OPTION_PROFILE, 1)
    for step in range(2):
        batch = batches[0] if batches is not None else workloads.batch(spec, seed=7, step=step)
        idx, off, psw = to_device(batch, index_dtype=idt)
        G = workloads.grad_output(spec, seed=7, step=step, device="cuda")
        ra, rb = gpu_runs(a, batch.N), gpu_runs(b, batch.N)
        _update(a, spec, idx, off, psw, G, ra, grouped)
        _update(b, spec, idx, off, psw, G, rb, grouped)
        torch.cuda.synchronize()
        if step == 0:
            used = _stages(a.op)
            assert "bucket_sort_rle" in used, f"{name}: bucket path not taken ({used})"
            assert "rle_kernel" not in used
            scatter = _linearize_tiles(spec) <= 256
            assert ("radix_pass" in used) == (not scatter), f"{name}: {used}"
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


def _per_table_batches():
    """Tables of different widths (short runs in per-table lane groups) where some tables get
    no lookup at all: the first and last table, one in the middle; one table whose lookups
    are a single row (one long run); and a batch whose runs all sit in one table."""
    rng = np.random.default_rng(41)
    T, B = 5, 96
    # table 0: empty; table 1: random; table 2: empty; table 3: one row 700 times; table 4: empty
    bags = [[[] for _ in range(B)] for _ in range(T)]
    for b in range(B):
        bags[1][b] = list(rng.integers(0, 300, rng.integers(0, 12)))
    hot = np.array_split(np.full(700, 17), B)
    for b in range(B):
        bags[3][b] = list(hot[b])
    only = [[[] for _ in range(B)] for _ in range(T)]
    for b in range(B):
        only[2][b] = list(rng.integers(0, 800, rng.integers(1, 9)))
    return _hand_batch(T, B, bags), _hand_batch(T, B, only)


@pytest.mark.parametrize("opt", ["sgd", "rowwise_adagrad"])
def test_per_table_groups_with_empty_tables(opt):
    spec = workloads.custom([500, 300, 800, 200, 64], [32, 256, 64, 128, 16], "bf16", B=96,
                            optimizer=opt, key=240)
    b1, b2 = _per_table_batches()
    parity(spec, seed=10, steps=2, batches=[b1, b2])


def test_sort_option_is_checked():
    spec = workloads.config(1)
    pb = make_problem(spec, seed=0)
    with pytest.raises(tbe.TBEError):
        pb.op.set_option(tbe.OPTION_SORT, 2)
    pb.op.set_option(tbe.OPTION_SORT, 1)
    pb.op.set_option(tbe.OPTION_SORT, 0)
    pb.op.close()


def _uniform_batch(E, B, n, seed):
    """One table, n uniform ids spread over B bags (ragged)."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, n)
    cuts = np.sort(rng.integers(0, n + 1, B - 1))
    off = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    return workloads.Batch(ids.astype(np.int64), off, None)


@pytest.mark.parametrize("E,n", [(1 << 20, 1 << 20), (1 << 20, (1 << 20) + 1),
                                 ((1 << 20) + 1, 1 << 19)],
                         ids=["20bit-2^20-lookups", "20bit-2^20+1-lookups", "21bit-ids"])
def test_path_boundaries(E, n):
    """Both sides of the bucket path's limits: 2^20 lookups (bucket path) and one more (counted
    LSD passes and the RLE kernel); ids of 20 bits (two digits) and of 21 bits (three LSD
    passes).  Runs bit-exact and sampled updates against the reference."""
    spec = workloads.custom([E], [16], "f32", B=4096, optimizer="rowwise_adagrad", key=250)
    batch = _uniform_batch(E, 4096, n, 51)
    pb = make_problem(spec, seed=11, batch=batch)
    pb.op.set_option(tbe.OPTION_PROFILE, 1)
    G = workloads.grad_output(spec, seed=11, step=0, device="cuda")
    runs = gpu_runs(pb, n)
    pb.op.backward_update(spec.B, pb.idx, pb.off, None, G, spec.lr, spec.eps, runs)
    torch.cuda.synchronize()
    used = _stages(pb.op)
    bucket = E == (1 << 20) and n <= (1 << 20)
    assert ("bucket_sort_rle" in used) == bucket, used
    assert ("rle_kernel" in used) == (not bucket), used
    # more than 2^20 lookups: counted passes (count, scan, place) and a counted
    # run-length encoding, no look-back
    counted = n > (1 << 20)
    assert ("radix_count" in used) == counted and ("radix_scan" in used) == counted, used
    assert ("rle_count" in used) == counted, used
    # up to 2^20 lookups the segment kernel finishes the long runs itself
    assert ("seg_finalize" in used) == counted, used
    pb.op.close()
    parity(spec, seed=12, steps=1, batches=[batch], bag_sample=500, row_sample=2000)


def test_counted_single_pass_with_records():
    """More than 2^20 lookups on 7-bit ids (one counted pass), mean pooling with per-sample
    weights (sorted values are lookup ids with side records): runs bit-exact and sampled
    updates against the reference."""
    spec = workloads.custom([100, 20], [16, 32], "f32", B=40000, lengths=("uniform_int", 20, 35),
                            index_dist=("zipf", 1.2), pooling="mean", psw=True,
                            optimizer="rowwise_adagrad", key=252)
    pb = make_problem(spec, seed=13)
    assert pb.batch.indices.size > (1 << 20)
    pb.op.set_option(tbe.OPTION_PROFILE, 1)
    G = workloads.grad_output(spec, seed=13, step=0, device="cuda")
    runs = gpu_runs(pb, pb.batch.indices.size)
    pb.op.backward_update(spec.B, pb.idx, pb.off, pb.psw, G, spec.lr, spec.eps, runs)
    torch.cuda.synchronize()
    used = [name for name, _ in pb.op.stage_times()]
    assert used.count("radix_count") == 1 and "rle_count" in used, used
    pb.op.close()
    parity(spec, seed=13, steps=2, bag_sample=3000)
