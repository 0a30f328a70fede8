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
