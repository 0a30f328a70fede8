"""The backward's grouping done during the forward (tbe_forward_group) and reused by
tbe_backward_update_grouped: kimbodo.com/?p=28372, "Kimbodo Engineering Perspective" (the
transpose, sort and run-length encoding can move into the forward).  Same results as the
plain calls, bit for bit, and parity with the CPU reference."""
import numpy as np
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import make_problem, rows_of, to_device
from test_gpu_parity import UNIT, parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("spec", [UNIT[0], UNIT[2], UNIT[4], UNIT[10]],
                         ids=["f32", "f16-mean", "bf16-mean-psw", "long-bags"])
def test_grouped_parity(spec):
    parity(spec, seed=11, steps=2, grouped=True)


def test_grouped_parity_8_tables_100k_rows_zipf():
    parity(workloads.config(2), seed=0, steps=2, bag_sample=3000, row_sample=3000, grouped=True)


def test_grouped_int32_ids():
    parity(UNIT[4], seed=12, steps=2, index_dtype=torch.int32, grouped=True)


def _grouped_vs_plain(spec, seed, steps, flags=0, index_dtype=torch.int64):
    """Two handles on identical weights and state: one with the plain calls, one with
    forward_group + backward_update_grouped.  Outputs, weights and state must be
    identical after every step."""
    a = make_problem(spec, seed=seed, flags=flags)
    b = make_problem(spec, seed=seed, flags=flags)
    for step in range(steps):
        batch = workloads.batch(spec, seed=seed, step=step)
        idx, off, psw = to_device(batch, index_dtype)
        G = workloads.grad_output(spec, seed=seed, step=step, device="cuda")
        ya = a.op.forward(spec.B, idx, off, psw)
        yb = b.op.forward_group(spec.B, idx, off, psw)
        a.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        b.op.backward_update_grouped(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"step {step}: forward"
        assert torch.equal(a.W, b.W), f"step {step}: weights"
        if a.state is not None:
            assert torch.equal(a.state, b.state), f"step {step}: state"
    a.op.close()
    b.op.close()


@pytest.mark.parametrize("every_table", [False, True], ids=["mixed", "all-routed"])
def test_grouped_with_count_matrix_routing(every_table):
    """Tables routed to the count-matrix forward are pooled by their own kernel; the fused
    launch then pools only the others (none when every table is routed) and still
    linearizes the whole batch."""
    if every_table:
        spec = workloads.custom([64, 700, 1000], [64, 32, 16], "bf16", B=257,
                                lengths=("uniform_int", 0, 30), key=420)
    else:
        spec = workloads.custom([64, 5000, 1000], [64, 32, 48], "bf16", B=257,
                                lengths=("uniform_int", 0, 30), key=421)
    _grouped_vs_plain(spec, seed=13, steps=2, flags=tbe.FLAG_HISTOGRAM)


@pytest.mark.parametrize("n", [2, 4])
def test_grouped_matches_plain_bit_for_bit(n):
    """Two handles on identical weights and state, three steps each: one with the plain
    calls, one with forward_group + backward_update_grouped.  Outputs, weights and state
    must be identical."""
    spec = workloads.config(n)
    a = make_problem(spec, seed=1)
    b = make_problem(spec, seed=1)
    for step in range(3):
        batch = workloads.batch(spec, seed=1, step=step)
        idx, off, psw = to_device(batch)
        G = workloads.grad_output(spec, seed=1, step=step, device="cuda")
        ya = a.op.forward(spec.B, idx, off, psw)
        yb = b.op.forward_group(spec.B, idx, off, psw)
        a.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        b.op.backward_update_grouped(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"step {step}: forward"
        assert torch.equal(a.W, b.W), f"step {step}: weights"
        if a.state is not None:
            assert torch.equal(a.state, b.state), f"step {step}: state"
    a.op.close()
    b.op.close()


def test_grouped_empty_batch_and_small_workspace():
    spec = UNIT[0]
    pb = make_problem(spec, seed=2)
    Y = torch.empty((spec.B, spec.sum_dims), device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tbe.TBEError, match="WORKSPACE_TOO_SMALL"):
        tbe.tbe_forward_group(pb.op.handle, spec.B, pb.idx, pb.off, None, Y, small)
    # B = 0: nothing to do
    tbe.tbe_forward_group(pb.op.handle, 0, pb.idx[:0], pb.off[:1], None, Y, small)
    torch.cuda.synchronize()
    pb.op.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n", [3, 5])
def test_grouped_matches_plain_bit_for_bit_large_batches(n):
    """The same on the mixed-width batch (5.2 M lookups: mean pooling with per-sample
    weights, per-table lane groups, LSD passes) and the many-small-tables batch (16.8 M
    lookups: the stand-alone linearize after the pooled lookup), two steps."""
    spec = workloads.config(n)
    print(f"[grouped-vs-plain] {spec.name}", flush=True)
    a = make_problem(spec, seed=1)
    b = make_problem(spec, seed=1)
    for step in range(2):
        batch = workloads.batch(spec, seed=1, step=step)
        idx, off, psw = to_device(batch)
        G = workloads.grad_output(spec, seed=1, step=step, device="cuda")
        ya = a.op.forward(spec.B, idx, off, psw)
        yb = b.op.forward_group(spec.B, idx, off, psw)
        a.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        b.op.backward_update_grouped(spec.B, idx, off, psw, G, spec.lr, spec.eps)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"step {step}: forward"
        assert torch.equal(a.W, b.W), f"step {step}: weights"
        if a.state is not None:
            assert torch.equal(a.state, b.state), f"step {step}: state"
        print(f"  step {step} identical", flush=True)
    a.op.close()
    b.op.close()


def _workspace(op, B, n):
    need = tbe.tbe_backward_workspace_size(op.handle, B, n)
    return torch.empty(need, dtype=torch.uint8, device="cuda")


def test_grouped_pairs_interleaved_on_two_workspaces():
    """Two forward_group calls (on two workspaces) before their backward calls: a batch of
    about 270k lookups (bucket-local sort, whose run-length encoding queues the longer runs)
    and one of more than 2^20 lookups (LSD passes; the runs are queued in the backward).
    The long-run threshold changes between the forward and the backward of each pair; the
    grouping keeps the one in force at its forward.  Everything must equal the plain calls
    made at that threshold, bit for bit."""
    spec = workloads.custom([100_000] * 2, [64, 64], "f32", B=2048, lengths=("uniform_int", 1, 32),
                            index_dist=("zipf", 1.05), optimizer="rowwise_adagrad", key=430)
    big = workloads.custom([100_000] * 2, [64, 64], "f32", B=36_000, lengths=("uniform_int", 1, 32),
                           index_dist=("zipf", 1.05), optimizer="rowwise_adagrad", key=430)
    b1 = workloads.batch(spec, seed=2, step=0)
    b2 = workloads.batch(big, seed=2, step=1)
    assert b1.N <= (1 << 20) < b2.N
    a = make_problem(spec, seed=2)     # plain calls
    g = make_problem(spec, seed=2)     # grouped pairs
    d1, d2 = to_device(b1), to_device(b2)
    G1 = workloads.grad_output(spec, seed=2, step=0, device="cuda")
    G2 = workloads.grad_output(big, seed=2, step=1, device="cuda")
    g.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 1)   # room for any threshold
    ws1, ws2 = _workspace(g.op, spec.B, b1.N), _workspace(g.op, big.B, b2.N)
    g.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 256)
    Y1 = torch.empty((spec.B, spec.sum_dims), device="cuda")
    Y2 = torch.empty((big.B, big.sum_dims), device="cuda")
    # grouped: both forwards first, the threshold changed in between
    tbe.tbe_forward_group(g.op.handle, spec.B, d1[0], d1[1], None, Y1, ws1)
    g.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 64)
    tbe.tbe_forward_group(g.op.handle, big.B, d2[0], d2[1], None, Y2, ws2)
    g.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 1 << 30)
    tbe.tbe_backward_update_grouped(g.op.handle, spec.B, d1[0], d1[1], None, G1, spec.lr,
                                    spec.eps, ws1)
    tbe.tbe_backward_update_grouped(g.op.handle, big.B, d2[0], d2[1], None, G2, big.lr,
                                    big.eps, ws2)
    # plain: the same forwards (before any update), then the updates at those thresholds
    ya1 = a.op.forward(spec.B, d1[0], d1[1])
    ya2 = a.op.forward(big.B, d2[0], d2[1])
    a.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 256)
    a.op.backward_update(spec.B, d1[0], d1[1], None, G1, spec.lr, spec.eps)
    a.op.set_option(tbe.OPTION_LONG_RUN_THRESHOLD, 64)
    a.op.backward_update(big.B, d2[0], d2[1], None, G2, big.lr, big.eps)
    torch.cuda.synchronize()
    assert torch.equal(ya1, Y1) and torch.equal(ya2, Y2)
    assert torch.equal(a.W, g.W) and torch.equal(a.state, g.state)
    a.op.close()
    g.op.close()


def test_grouped_backward_rejects_a_batch_it_did_not_group():
    """The grouped backward needs a forward_group of the same batch buffers in the same
    workspace; otherwise it returns TBE_ERR_INVALID_ARGUMENT with nothing enqueued, and a
    grouping serves one backward call."""
    spec = UNIT[0]
    pb = make_problem(spec, seed=5)
    W0 = pb.W.clone()
    G = workloads.grad_output(spec, seed=5, step=0, device="cuda")
    ws = _workspace(pb.op, spec.B, pb.batch.N)
    Y = torch.empty((spec.B, spec.sum_dims), device="cuda")

    def grouped_backward(idx, off, B=spec.B):
        tbe.tbe_backward_update_grouped(pb.op.handle, B, idx, off, None, G, spec.lr, spec.eps, ws)

    with pytest.raises(tbe.TBEError, match="INVALID_ARGUMENT"):   # nothing grouped yet
        grouped_backward(pb.idx, pb.off)
    tbe.tbe_forward_group(pb.op.handle, spec.B, pb.idx, pb.off, None, Y, ws)
    with pytest.raises(tbe.TBEError, match="INVALID_ARGUMENT"):   # other id buffer
        grouped_backward(pb.idx.clone(), pb.off)
    with pytest.raises(tbe.TBEError, match="INVALID_ARGUMENT"):   # other offsets buffer
        grouped_backward(pb.idx, pb.off.clone())
    torch.cuda.synchronize()
    assert torch.equal(pb.W, W0)
    grouped_backward(pb.idx, pb.off)                               # the matching call
    torch.cuda.synchronize()
    assert not torch.equal(pb.W, W0)
    with pytest.raises(tbe.TBEError, match="INVALID_ARGUMENT"):   # the grouping is used up
        grouped_backward(pb.idx, pb.off)
    # a plain backward on the workspace discards a grouping left in it
    tbe.tbe_forward_group(pb.op.handle, spec.B, pb.idx, pb.off, None, Y, ws)
    tbe.tbe_backward_update(pb.op.handle, spec.B, pb.idx, pb.off, None, G, spec.lr, spec.eps, ws)
    with pytest.raises(tbe.TBEError, match="INVALID_ARGUMENT"):
        grouped_backward(pb.idx, pb.off)
    torch.cuda.synchronize()
    pb.op.close()
