"""GPU parity of the HIP library (through its C ABI) against the CPU reference.

Forward pooling over all tables with optional per-sample weights and fp32
accumulation, and the fused backward (linearize, sort, run-length encode,
segment reduce, one optimizer update per touched row): kimbodo.com/?p=28372,
"What Happened" and "Kimbodo Engineering Perspective".  Comparison rules are
documented in gpu_check.py.
"""
import numpy as np
import pytest
import torch

import oracle
import table_embedding_bag_amd as tbe
import workloads
from gpu_check import (carry_deviation, check_forward, check_runs, check_update, guarded_empty,
                       make_problem, reference_update, rows_of, run_step, to_device,
                       untouched_identical)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def parity(spec, seed=0, steps=2, bag_sample=None, row_sample=None, index_dtype=torch.int64,
           threshold=None, batches=None, flags=0, grouped=False):
    """Forward and backward_update for `steps` steps, each checked against the reference,
    which advances its own copy of weights and state."""
    _say(f"[parity] {spec.name} dtype={spec.dtype} seed={seed} thr={threshold} flags={flags}")
    pb = make_problem(spec, seed=seed, index_dtype=index_dtype,
                      batch=None if batches is None else batches[0], flags=flags)
    if threshold is not None:
        pb.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, threshold)
    W_host = workloads.storage_numpy(pb.W).copy()
    st_host = np.zeros(spec.sum_rows, np.float32) if pb.state is not None else None
    rng = np.random.default_rng(seed + 99)
    dev = np.zeros(spec.sum_rows)   # allowed |W_gpu - W_ref| per row, carried across steps
    report = {}
    for step in range(steps):
        if step > 0:
            pb.batch = batches[step] if batches is not None else workloads.batch(spec, seed=seed, step=step)
            pb.idx, pb.off, pb.psw = to_device(pb.batch, index_dtype)
        nbags = spec.T * spec.B
        sample = None
        if bag_sample is not None and bag_sample < nbags:
            sample = np.unique(np.concatenate([
                rng.choice(nbags, bag_sample, replace=False),
                np.arange(spec.T) * spec.B, np.arange(1, spec.T + 1) * spec.B - 1]))
        ybuf, Y = guarded_empty((spec.B, spec.sum_dims), torch.float32)
        if grouped:
            pb.op.forward_group(spec.B, pb.idx, pb.off, pb.psw, out=Y)
        else:
            pb.op.forward(spec.B, pb.idx, pb.off, pb.psw, out=Y)
        torch.cuda.synchronize()
        pb.check_guards(ybuf)
        report[f"fwd{step}"] = check_forward(pb, Y, W_host, sample, dev)
        _say(f"  step {step}: forward ok (max rel {report[f'fwd{step}']:.2e})")

        G = workloads.grad_output(spec, seed=seed, step=step, device="cuda")
        # rows this step leaves alone, as the GPU holds them before the step
        ref_uniq, _ = oracle.runs(spec.rows, spec.B, pb.batch.indices, pb.batch.offsets)
        untouched = np.setdiff1d(np.arange(spec.sum_rows), ref_uniq, assume_unique=True)
        if untouched.size > 20000:
            untouched = np.sort(rng.choice(untouched, 20000, replace=False))
        gpu_before = rows_of(spec, pb.W, untouched)
        gpu_st_before = pb.state.cpu().numpy() if pb.state is not None else None
        runs = run_step(pb, G, grouped=grouped)
        uniq, cnt = check_runs(pb, runs)
        _say(f"  step {step}: runs ok (U={uniq.size}, max run {cnt.max() if cnt.size else 0})")
        if row_sample is not None and uniq.size > row_sample:
            hot = uniq[np.argsort(cnt)[-50:]]
            sel = np.unique(np.concatenate([rng.choice(uniq, row_sample, replace=False), hot,
                                            uniq[:5], uniq[-5:]]))
        else:
            sel = uniq
        before_all = rows_of(spec, W_host, uniq)
        reference_update(pb, W_host, st_host, G.cpu().numpy())
        after_all = rows_of(spec, W_host, uniq)
        st_gpu = pb.state.cpu().numpy() if pb.state is not None else None
        counts = dict(zip(uniq.tolist(), cnt.tolist()))
        before_sel = before_all if sel is uniq else _subset(spec, before_all, uniq, sel)
        report[f"upd{step}"] = check_update(spec, sel, before_sel,
                                            rows_of(spec, W_host, sel), rows_of(spec, pb.W, sel), dev,
                                            st_host, st_gpu, counts)
        carry_deviation(spec, dev, uniq, before_all, after_all)
        # rows nobody looked up in this step stay bit-identical
        if untouched.size:
            untouched_identical(spec, gpu_before, rows_of(spec, pb.W, untouched),
                                gpu_st_before, st_gpu, untouched)
        pb.check_guards()
        _say(f"  step {step}: update ok (worst {report[f'upd{step}']:.3f})")
    pb.op.close()
    return report


def _subset(spec, rows: dict, ids, sel):
    """Rows of `sel` (a sorted subset of sorted `ids`) out of a rows_of(ids) dict."""
    from gpu_check import layout
    _, roff, _ = layout(spec)
    tab_ids = np.searchsorted(roff, ids, side="right") - 1
    out = {}
    for t in np.unique(np.searchsorted(roff, sel, side="right") - 1):
        mine = ids[tab_ids == t]
        want = sel[(sel >= roff[t]) & (sel < roff[t + 1])]
        out[int(t)] = rows[int(t)][np.searchsorted(mine, want)]
    return out


# --------------------------------------------------------------------------
# the page's worked example and small unit cases
# --------------------------------------------------------------------------

def test_worked_example_bit_exact():
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    E, D = 16, 8
    Wn = (np.arange(E)[:, None] + np.arange(D)[None, :] / 4.0).astype(np.float32)
    W = torch.from_numpy(Wn.reshape(-1)).cuda()
    op = tbe.TBE([E], [D], W)
    idx = torch.tensor(ex["indices"], dtype=torch.int64, device="cuda")
    off = torch.tensor(ex["offsets"], dtype=torch.int64, device="cuda")
    Y = op.forward(len(ex["offsets"]) - 1, idx, off).cpu().numpy()
    for b, bag in enumerate(ex["bags"]):
        assert np.array_equal(Y[b], Wn[bag].sum(axis=0))
    op.close()


UNIT = [
    workloads.custom([50, 7, 300], [8, 4, 16], "f32", B=33, lengths=("uniform_int", 0, 9), key=201),
    workloads.custom([50, 7, 300], [8, 16, 32], "bf16", B=33, lengths=("uniform_int", 0, 9), key=202,
                     optimizer="rowwise_adagrad"),
    workloads.custom([20, 90], [64, 8], "f16", B=70, lengths=("uniform_int", 0, 40),
                     index_dist=("zipf", 1.2), pooling="mean", optimizer="rowwise_adagrad", key=203),
    workloads.custom([40, 13, 9], [4, 12, 64], "f32", B=65, lengths=("uniform_int", 0, 8), psw=True,
                     key=204),
    workloads.custom([40, 13, 9], [8, 24, 64], "bf16", B=65, lengths=("uniform_int", 0, 8), psw=True,
                     pooling="mean", optimizer="rowwise_adagrad", key=205),
    # dims that are not whole 16-byte chunks: one element per lane
    workloads.custom([30, 11], [6, 3], "f32", B=17, lengths=("uniform_int", 0, 7), key=206,
                     optimizer="rowwise_adagrad"),
    workloads.custom([30, 11], [6, 10], "bf16", B=17, lengths=("uniform_int", 0, 7), key=207,
                     psw=True, pooling="mean"),
    # wide rows: chunk sets per lane in both directions
    workloads.custom([100, 60], [512, 1024], "f32", B=9, lengths=("uniform_int", 1, 20), key=208,
                     optimizer="rowwise_adagrad"),
    workloads.custom([100, 60], [520, 96], "f16", B=9, lengths=("uniform_int", 1, 20), key=209),
    workloads.custom([100], [300], "bf16", B=9, lengths=("uniform_int", 1, 20), key=210),
    # long bags (a whole wave per bag, several index chunks)
    workloads.custom([1000], [128], "f32", B=40, lengths=("uniform_int", 60, 300), key=211,
                     index_dist=("zipf", 1.1), optimizer="rowwise_adagrad"),
]


@pytest.mark.parametrize("spec", UNIT, ids=lambda s: f"{s.key}-{s.dtype}-{s.pooling}-psw{int(s.psw)}-{s.optimizer}")
def test_unit_parity(spec):
    parity(spec, seed=1, steps=2)


@pytest.mark.parametrize("spec", [UNIT[0], UNIT[4]], ids=["f32", "bf16-mean-psw"])
def test_int32_indices(spec):
    parity(spec, seed=2, steps=1, index_dtype=torch.int32)


# more tables than the segment kernels stage in LDS (256): table metadata is then read from
# global memory
_rng = np.random.default_rng(301)
MANY = [
    workloads.custom(_rng.integers(3, 60, 300), [(4, 8, 16, 12)[t % 4] for t in range(300)], "f32",
                     B=7, lengths=("uniform_int", 0, 6), pooling="mean", psw=True,
                     optimizer="rowwise_adagrad", key=301),
    workloads.custom(_rng.integers(3, 60, 270), [(8, 16, 32)[t % 3] for t in range(270)], "bf16",
                     B=5, lengths=("uniform_int", 0, 9), index_dist=("zipf", 1.3), key=302),
]


@pytest.mark.parametrize("spec", MANY, ids=["300-f32-mean-psw-adagrad", "270-bf16-sum-sgd"])
def test_many_tables(spec):
    parity(spec, seed=3, steps=2)


def test_many_tables_grouped():
    parity(MANY[0], seed=4, steps=2, grouped=True)


def _hand_batch(T, B, bags):
    """bags: list (per table) of lists (per bag) of row ids."""
    lens = [len(b) for tb in bags for b in tb]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = np.array([x for tb in bags for b in tb for x in b], dtype=np.int64)
    return workloads.Batch(idx, off, None)


def test_run_length_boundaries_and_long_runs():
    # rows hit exactly 255 / 256 / 257 times straddle the long-run threshold; one row
    # hit 20000 times needs more than 32 chunk partials (the two-level combine).
    E, D, B = 64, 32, 400
    rng = np.random.default_rng(3)
    hits = [3] * 255 + [7] * 256 + [9] * 257 + [11] * 20000 + list(rng.integers(0, E, 3000))
    hits = rng.permutation(np.array(hits))
    per_bag = np.array_split(hits, B)
    batch = _hand_batch(1, B, [[list(b) for b in per_bag]])
    for opt in ("sgd", "rowwise_adagrad"):
        spec = workloads.custom([E], [D], "f32", B=B, optimizer=opt, key=220)
        for thr in (None, 1, 1 << 30):
            parity(spec, seed=4, steps=1, threshold=thr, batches=[batch])


@pytest.mark.parametrize("dtype,D", [("f32", 32), ("bf16", 128)])
def test_very_long_runs_finish_in_pieces(dtype, D):
    # Runs of at least 128 chunk partials (32 768 lookups) are finished in pieces of 64
    # chunks, the last taking the remainder: rows hit 32 512 times (127 chunks, one
    # workgroup), 32 768 (two pieces of 64), 33 000 (64 + 65) and 50 000 times
    # (64 + 64 + 68).  Two steps on one handle, plain and grouped calls, and the same
    # result bit for bit on a second handle.
    E, B = 64, 512
    rng = np.random.default_rng(7)
    hits = [5] * 32512 + [13] * 32768 + [21] * 33000 + [29] * 50000 + list(rng.integers(0, E, 4000))
    batches = []
    for step in range(2):
        h = rng.permutation(np.array(hits))
        batches.append(_hand_batch(1, B, [[list(b) for b in np.array_split(h, B)]]))
    for opt in ("sgd", "rowwise_adagrad"):
        spec = workloads.custom([E], [D], dtype, B=B, optimizer=opt, key=225)
        parity(spec, seed=6, steps=2, batches=batches)
    parity(spec, seed=6, steps=2, batches=batches, grouped=True)
    a = make_problem(spec, seed=8, batch=batches[0])
    b = make_problem(spec, seed=8, batch=batches[0])
    G = workloads.grad_output(spec, seed=8, step=0, device="cuda")
    for pb in (a, b):
        pb.op.backward_update(B, pb.idx, pb.off, None, G, spec.lr, spec.eps)
    torch.cuda.synchronize()
    assert torch.equal(a.W, b.W) and torch.equal(a.state, b.state)
    a.op.close()
    b.op.close()


@pytest.mark.parametrize("extra", [0, 320_000], ids=["finished-in-items", "finalize-launch"])
def test_many_long_runs_finish_once_each(extra):
    # 250 rows hit 256 to 12 000 times (1 to 47 chunk partials) and two rows hit 33 000 and
    # 40 000 times (pieces of 64 chunks), among uniform lookups: about 770k lookups, so the
    # workgroup that stores a run's last partial finishes it inside the segment kernel; with
    # 320k more uniform lookups the batch passes 2^20 and a separate launch finishes the runs.
    # Both against the reference (every row updated once), and three handles bit-identical.
    E, D, B = 3000, 64, 2048
    rng = np.random.default_rng(17)
    counts = np.exp(rng.uniform(np.log(256), np.log(12000), 250)).astype(np.int64)
    hot = rng.choice(E, 252, replace=False)
    hits = np.concatenate([np.repeat(hot[:250], counts), np.repeat(hot[250], 33000),
                           np.repeat(hot[251], 40000), rng.integers(0, E, 20000 + extra)])
    hits = rng.permutation(hits)
    assert (len(hits) <= (1 << 20)) == (extra == 0)
    batch = _hand_batch(1, B, [[list(b) for b in np.array_split(hits, B)]])
    spec = workloads.custom([E], [D], "f32", B=B, optimizer="rowwise_adagrad", key=226)
    parity(spec, seed=9, steps=1, batches=[batch])
    outs = []
    G = workloads.grad_output(spec, seed=9, step=0, device="cuda")
    for _ in range(3):
        pb = make_problem(spec, seed=9, batch=batch)
        pb.op.backward_update(B, pb.idx, pb.off, None, G, spec.lr, spec.eps)
        torch.cuda.synchronize()
        outs.append((pb.W.clone(), pb.state.clone()))
        pb.op.close()
    for W, st in outs[1:]:
        assert torch.equal(W, outs[0][0]) and torch.equal(st, outs[0][1])


@pytest.mark.parametrize("cycle", [(2, 0, 4, 2), (2, 1, 3, 2), (8,)], ids=["with-empty", "uneven", "even"])
def test_linearize_tiles_whose_lengths_sum_evenly(cycle):
    # Bag lengths cycling (2, 0, 4, 2) or (2, 1, 3, 2) make every tile of 128 bags hold
    # 128 times its first bag's length although the bags differ (so the interpolated bag
    # slot is often wrong and must be caught); (8,) is the truly even case.
    T, B, E = 2, 1024, 300
    rng = np.random.default_rng(9)
    bags = [[list(rng.integers(0, E, cycle[b % len(cycle)])) for b in range(B)] for t in range(T)]
    batch = _hand_batch(T, B, bags)
    spec = workloads.custom([E, E], [32, 32], "f32", B=B, optimizer="rowwise_adagrad", key=226)
    parity(spec, seed=10, steps=1, batches=[batch])
    parity(spec, seed=10, steps=1, batches=[batch], grouped=True)
    parity(spec, seed=10, steps=1, batches=[batch], index_dtype=torch.int32)


def test_dyadic_sgd_is_bit_exact():
    # with dyadic weights, gradients and learning rate every sum is exact in any order
    E, D, B = 40, 16, 300
    rng = np.random.default_rng(5)
    spec = workloads.custom([E, E], [D, D], "f32", B=B, lengths=("uniform_int", 0, 12),
                            index_dist=("zipf", 1.3), key=230, lr=0.25)
    batch = workloads.batch(spec, seed=5)
    Wn = (rng.integers(-64, 64, spec.num_weights) / 64.0).astype(np.float32)
    Gn = (rng.integers(-8, 8, (B, spec.sum_dims)) / 8.0).astype(np.float32)
    W = torch.from_numpy(Wn).cuda()
    G = torch.from_numpy(Gn).cuda()
    op = tbe.TBE(spec.rows, spec.dims, W)
    idx, off, _ = to_device(batch)
    Y = op.forward(B, idx, off).cpu().numpy()
    Yr = oracle.forward(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, Wn, B, batch.indices,
                        batch.offsets)
    assert np.array_equal(Y, Yr)
    for thr in (1, 256, 1 << 30):
        W.copy_(torch.from_numpy(Wn))
        op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, thr)
        op.backward_update(B, idx, off, None, G, 0.25)
        Wr = Wn.copy()
        oracle.backward_update(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, oracle.OPT_SGD, Wr,
                               None, B, batch.indices, batch.offsets, None, Gn, 0.25, 0.0)
        assert np.array_equal(W.cpu().numpy(), Wr)
    op.close()


def test_empty_bags_and_empty_batch():
    spec = workloads.custom([10, 10], [8, 8], "f32", B=5, optimizer="rowwise_adagrad", key=240,
                            pooling="mean")
    W = workloads.weights(spec, 0, "cuda")
    W0 = W.clone()
    st = torch.zeros(spec.sum_rows, device="cuda")
    op = tbe.TBE(spec.rows, spec.dims, W, st, pooling="mean", optimizer="rowwise_adagrad")
    # all bags empty
    off = torch.zeros(2 * 5 + 1, dtype=torch.int64, device="cuda")
    idx = torch.zeros(0, dtype=torch.int64, device="cuda")
    Y = torch.full((5, 16), 7.0, device="cuda")
    op.forward(5, idx, off, out=Y)
    torch.cuda.synchronize()
    assert (Y == 0).all()
    G = torch.randn(5, 16, device="cuda")
    runs = (torch.zeros(1, dtype=torch.int32, device="cuda"),
            torch.zeros(1, dtype=torch.int32, device="cuda"),
            torch.full((1,), 5, dtype=torch.int32, device="cuda"))
    op.backward_update(5, idx, off, None, G, 0.1, runs=runs)
    torch.cuda.synchronize()
    assert int(runs[2].item()) == 0
    assert torch.equal(W, W0) and (st == 0).all()
    # B = 0 is a no-op
    op.forward(0, idx, torch.zeros(1, dtype=torch.int64, device="cuda"), out=Y)
    # one table all-empty, the other not
    batch = _hand_batch(2, 5, [[[], [], [], [], []], [[1, 2], [], [3], [3, 3, 9], []]])
    parity(spec, seed=0, steps=1, batches=[batch])
    op.close()


def test_validate_flag_rejects_bad_ids_without_touching_outputs():
    spec = workloads.custom([10, 20], [8, 8], "f32", B=4, key=250)
    W = workloads.weights(spec, 0, "cuda")
    W0 = W.clone()
    op = tbe.TBE(spec.rows, spec.dims, W, flags=tbe.FLAG_VALIDATE)
    idx = torch.tensor([1, 2, 10, 3, 19, 0], dtype=torch.int64, device="cuda")  # 10 is out of table 0
    off = torch.tensor([0, 2, 3, 3, 3, 4, 5, 6, 6], dtype=torch.int64, device="cuda")
    Y = torch.full((4, 16), 3.0, device="cuda")
    with pytest.raises(tbe.TBEError) as e:
        op.forward(4, idx, off, out=Y)
    assert e.value.status == 3
    assert (Y == 3.0).all()
    G = torch.ones(4, 16, device="cuda")
    with pytest.raises(tbe.TBEError):
        op.backward_update(4, idx, off, None, G, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(W, W0)
    idx[2] = 9
    op.forward(4, idx, off, out=Y)   # valid now
    bad_off = off.clone()
    bad_off[-1] = 5                  # offsets do not end at the id count
    with pytest.raises(tbe.TBEError):
        op.forward(4, idx, bad_off, out=Y)
    op.close()


def test_backward_is_deterministic():
    spec = workloads.config(2)
    spec = workloads.custom(spec.rows[:2], spec.dims[:2], "f32", B=1024, lengths=("uniform_int", 1, 32),
                            index_dist=("zipf", 1.3), optimizer="rowwise_adagrad", key=260)
    batch = workloads.batch(spec, seed=7)
    idx, off, _ = to_device(batch)
    G = workloads.grad_output(spec, seed=7, device="cuda")
    outs = []
    for _ in range(2):
        W = workloads.weights(spec, 7, "cuda")
        st = torch.zeros(spec.sum_rows, device="cuda")
        op = tbe.TBE(spec.rows, spec.dims, W, st, optimizer="rowwise_adagrad")
        op.backward_update(spec.B, idx, off, None, G, 0.01)
        torch.cuda.synchronize()
        outs.append((W.clone(), st.clone()))
        op.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# --------------------------------------------------------------------------
# the five benchmark workloads, two optimizer steps each
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_parity(n):
    spec = workloads.config(n)
    big = n >= 3
    parity(spec, seed=0, steps=2, bag_sample=20000 if big else None,
           row_sample=50000 if big else None)
