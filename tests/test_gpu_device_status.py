"""Failure reporting of the backward: every wait of one workgroup for another in the
grouping (the sort's and the run-length encoding's look-backs) is bounded by a per-handle
spin limit.  A wait that gives up must not fault, hang or update anything, and the caller
must learn of it (tbe_check_device_status, or the call's own status under
TBE_FLAG_VALIDATE).  The condition is forced from the host with a spin limit of 0, under
which every such wait gives up at once; every kernel still runs to its end."""
import numpy as np
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import (check_runs, check_update, gpu_runs, make_problem, reference_update,
                       rows_of, to_device)

pytestmark = pytest.mark.gpu

DEVICE_WAIT = 7

# 2 x 2048 bags of 1..32 lookups (about 68k lookups: 17 radix tiles, 33 bucket windows)
SPEC = workloads.custom([100_000, 100_000], [128, 128], "f32", B=2048,
                        lengths=("uniform_int", 1, 32), index_dist=("zipf", 1.05),
                        optimizer="rowwise_adagrad", key=510)


def _say(*a):
    print(*a, flush=True)


def _one_step_matches_reference(pb, seed):
    """A backward_update on the handle's current weights matches the CPU reference."""
    spec = pb.spec
    W_host = pb.W.cpu().numpy().copy()
    st_host = pb.state.cpu().numpy().copy()
    G = workloads.grad_output(spec, seed=seed, step=5, device="cuda")
    runs = gpu_runs(pb, pb.batch.N)
    pb.op.backward_update(spec.B, pb.idx, pb.off, None, G, spec.lr, spec.eps, runs)
    torch.cuda.synchronize()
    uniq, cnt = check_runs(pb, runs)
    before = rows_of(spec, W_host, uniq)
    reference_update(pb, W_host, st_host, G.cpu().numpy())
    check_update(spec, uniq, before, rows_of(spec, W_host, uniq), rows_of(spec, pb.W, uniq),
                 np.zeros(spec.sum_rows), st_host, pb.state.cpu().numpy())


@pytest.mark.parametrize("grouped", [False, True], ids=["plain", "grouped"])
@pytest.mark.parametrize("sort", [0, 1], ids=["bucket-sort", "lsd-passes"])
def test_wait_that_gives_up_updates_nothing_and_is_reported(sort, grouped):
    _say(f"[device-status] sort={sort} grouped={grouped} N~68k")
    pb = make_problem(SPEC, seed=3)
    pb.op.set_option(tbe.OPTION_SORT, sort)
    pb.op.set_option(tbe.OPTION_SPIN_LIMIT, 0)
    W0, st0 = pb.W.clone(), pb.state.clone()
    G = workloads.grad_output(SPEC, seed=3, step=0, device="cuda")
    runs = gpu_runs(pb, pb.batch.N)
    if grouped:
        Y = pb.op.forward_group(SPEC.B, pb.idx, pb.off)
        pb.op.backward_update_grouped(SPEC.B, pb.idx, pb.off, None, G, SPEC.lr, SPEC.eps, runs)
    else:
        Y = pb.op.forward(SPEC.B, pb.idx, pb.off)
        pb.op.backward_update(SPEC.B, pb.idx, pb.off, None, G, SPEC.lr, SPEC.eps, runs)
    torch.cuda.synchronize()
    assert torch.isfinite(Y).all()
    assert int(runs[2].item()) == -1                     # the call says it gave up
    assert torch.equal(pb.W, W0) and torch.equal(pb.state, st0)
    with pytest.raises(tbe.TBEError) as e:
        pb.op.check_device_status()
    assert e.value.status == DEVICE_WAIT
    pb.op.check_device_status()                          # the mark was cleared
    # the default limit again: the same handle and workspace work normally
    pb.op.set_option(tbe.OPTION_SPIN_LIMIT, 1 << 20)
    _one_step_matches_reference(pb, seed=3)
    pb.op.check_device_status()
    pb.op.close()


def test_validate_flag_returns_the_failure_from_the_call():
    _say("[device-status] validate flag")
    pb = make_problem(SPEC, seed=4, flags=tbe.FLAG_VALIDATE)
    pb.op.set_option(tbe.OPTION_SPIN_LIMIT, 0)
    W0, st0 = pb.W.clone(), pb.state.clone()
    G = workloads.grad_output(SPEC, seed=4, step=0, device="cuda")
    with pytest.raises(tbe.TBEError) as e:
        pb.op.backward_update(SPEC.B, pb.idx, pb.off, None, G, SPEC.lr, SPEC.eps)
    assert e.value.status == DEVICE_WAIT
    torch.cuda.synchronize()
    assert torch.equal(pb.W, W0) and torch.equal(pb.state, st0)
    pb.op.check_device_status()                          # the call already cleared the mark
    pb.op.set_option(tbe.OPTION_SPIN_LIMIT, 1 << 20)
    _one_step_matches_reference(pb, seed=4)
    pb.op.close()


def test_spin_limit_option_checks_its_value():
    pb = make_problem(workloads.custom([10], [8], "f32", B=2, key=511), seed=0)
    for bad in (-1, 1 << 31):
        with pytest.raises(tbe.TBEError):
            pb.op.set_option(tbe.OPTION_SPIN_LIMIT, bad)
    pb.op.close()
