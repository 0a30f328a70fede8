"""The pooled lookup of small tables from LDS (TBE_OPTION_LDS_FORWARD; the gather and pooling
of kimbodo.com/?p=28372, "What Happened", with each small table staged in a CU's local memory).

It keeps the gather kernel's partial sums and their fold, so its output must equal the gather
kernel's bit for bit (option 0), on tables that take the LDS path alone or next to tables that
do not (too large, or of another row width), with fixed and ragged bags (bags longer than a
lane group's first round of ids), per-sample weights, mean pooling, int32 and int64 ids.  The
same cases are checked against the CPU reference."""
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import make_problem, to_device
from test_gpu_parity import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


CASES = [
    # every table from LDS (rows of 8 chunks), two partial sums per bag
    ("bf16-fixed-8", workloads.custom([64, 1024, 300, 1000], [64] * 4, "bf16", B=4096,
                                      lengths=("fixed", 8), key=270), torch.int64),
    # bags of 0..14 lookups (rounds past the first 8 ids), two partial sums, mean + weights
    ("f16-ragged-psw-mean", workloads.custom([200, 500, 64], [64, 64, 64], "f16", B=3000,
                                             lengths=("uniform_int", 0, 14),
                                             index_dist=("zipf", 1.1), pooling="mean", psw=True,
                                             key=271), torch.int32),
    # bags of 0..30 lookups: four partial sums, rows of 8 chunks
    ("bf16-ragged-4-sums", workloads.custom([300, 1000], [64, 64], "bf16", B=2048,
                                            lengths=("uniform_int", 0, 30), key=274), torch.int64),
    # tables of 1, 2 and 3 rows (every id is one of a few rows) with bags up to 30 long
    ("bf16-tiny-tables", workloads.custom([1, 2, 3], [64, 64, 64], "bf16", B=2048,
                                          lengths=("uniform_int", 0, 30), key=276), torch.int64),
    # rows of 4 chunks with weights and four partial sums
    ("bf16-dim32-psw-4-sums", workloads.custom([500, 200], [32, 32], "bf16", B=2048,
                                               lengths=("uniform_int", 0, 30), psw=True,
                                               key=275), torch.int32),
    # rows of 4 chunks (dim 32) and of 8 chunks (dims 64 and 40, the LDS ones) and a table
    # over 128 KB: the others take the gather kernel in the same call
    ("bf16-mixed-widths", workloads.custom([100, 700, 5000, 300, 90], [32, 32, 32, 64, 40],
                                           "bf16", B=2048, lengths=("uniform_int", 1, 12),
                                           key=272), torch.int64),
]


def _forward(pb, spec, lds):
    pb.op.set_option(tbe.OPTION_LDS_FORWARD, 1 if lds else 0)
    pb.op.set_option(tbe.OPTION_PROFILE, 1)
    tbe.tbe_stage_times(pb.op.handle)
    Y = pb.op.forward(spec.B, pb.idx, pb.off, pb.psw)
    torch.cuda.synchronize()
    used = {name for name, _ in tbe.tbe_stage_times(pb.op.handle)}
    pb.op.set_option(tbe.OPTION_PROFILE, 0)
    return Y, used


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lds_forward_equals_gather(case):
    name, spec, idt = case
    _say(f"[lds forward] {name}")
    pb = make_problem(spec, seed=3, index_dtype=idt)
    Yg, used_g = _forward(pb, spec, lds=False)
    Yl, used_l = _forward(pb, spec, lds=True)
    assert "fwd_lds_pool" in used_l and "fwd_lds_pool" not in used_g, (used_l, used_g)
    assert torch.equal(Yl, Yg), f"{name}: max |diff| {(Yl - Yg).abs().max().item()}"
    pb.op.close()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lds_forward_parity(case):
    name, spec, idt = case
    parity(spec, seed=4, steps=1, index_dtype=idt)


def test_lds_forward_full_small_table_workload():
    """64 bf16 tables of 64-1024 rows, 32768 bags of 8 lookups: LDS against the gather."""
    spec = workloads.config(5)
    pb = make_problem(spec, seed=5)
    Yg, _ = _forward(pb, spec, lds=False)
    Yl, used = _forward(pb, spec, lds=True)
    assert "fwd_lds_pool" in used
    assert torch.equal(Yl, Yg)
    # the grouped forward takes the same path on this batch
    Y2 = torch.empty_like(Yl)
    pb.op.forward_group(spec.B, pb.idx, pb.off, pb.psw, out=Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y2, Yl)
    pb.op.close()


def test_lds_forward_needs_enough_lookups_and_is_checked():
    """Too few lookups per table for the staging to pay, or bags too long for the partial
    sums the LDS kernel keeps: the gather kernel runs."""
    for rows, B, lengths, psw in (([1000, 800], 64, ("fixed", 4), False),
                                  ([300, 200], 2048, ("uniform_int", 20, 40), False),
                                  ([300, 200], 2048, ("uniform_int", 8, 16), True)):
        spec = workloads.custom(rows, [64, 64], "bf16", B=B, lengths=lengths, psw=psw, key=273)
        pb = make_problem(spec, seed=6)
        _, used = _forward(pb, spec, lds=True)
        assert "fwd_lds_pool" not in used and "fwd_gather_pool" in used, (rows, lengths, used)
        with pytest.raises(tbe.TBEError):
            pb.op.set_option(tbe.OPTION_LDS_FORWARD, 2)
        pb.op.close()
