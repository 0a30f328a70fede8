"""The forward's opt-in paths take their device scratch from the caller (the boundary
allocates only the handle's metadata block): the count-matrix forward's transposed tables
(kimbodo.com/?p=28372, "What Happened": small tables use a histogram and matrix-core path)
and the split bags' segment sums (same page, "Kimbodo Engineering Perspective": load
imbalance across lookups).  Through the C ABI: the size query, the errors of a missing,
misaligned or short scratch, and the same output bits as the binding's own scratch."""
import numpy as np
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import make_problem
from test_gpu_split_bags import _batches

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _raw_handle(spec, W, flags):
    dt = {"f32": tbe.F32, "f16": tbe.F16, "bf16": tbe.BF16}[spec.dtype]
    return tbe.tbe_create(spec.rows, spec.dims, dt, tbe.POOL_SUM, tbe.OPT_SGD, W, None, flags)


def _status(fn, *args):
    try:
        fn(*args)
        return 0
    except tbe.TBEError as e:
        return e.status


CASES = [
    ("split-bags", workloads.custom([5000, 3000], [128, 64], "f32", B=48, key=260),
     tbe.FLAG_SPLIT_BAGS),
    ("histogram", workloads.custom([300, 1000, 64], [64, 32, 128], "bf16", B=256,
                                   lengths=("uniform_int", 0, 40), key=270),
     tbe.FLAG_HISTOGRAM),
]


@pytest.mark.parametrize("name,spec,flags", CASES, ids=[c[0] for c in CASES])
def test_forward_scratch_is_the_callers(name, spec, flags):
    _say(f"[scratch] {name}")
    batches = _batches(spec, 21) if flags == tbe.FLAG_SPLIT_BAGS else None
    pb = make_problem(spec, seed=3, batch=batches[0] if batches else None, flags=flags)
    ref = pb.op.forward(spec.B, pb.idx, pb.off)   # the binding attaches its own scratch
    h = _raw_handle(spec, pb.W, flags)
    try:
        need = tbe.tbe_forward_scratch_size(h)
        assert need > 0
        out = torch.empty_like(ref)
        # no scratch attached: refused, nothing written
        out.fill_(7.0)
        assert _status(tbe.tbe_forward, h, spec.B, pb.idx, pb.off, None, out) == 4
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
        buf = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
        assert _status(tbe.tbe_set_forward_scratch, h, buf[1:], need) == 1   # misaligned
        assert _status(tbe.tbe_set_forward_scratch, h, buf, need - 1) == 4   # too small
        assert _status(tbe.tbe_set_forward_scratch, h, None, 16) == 1        # NULL with bytes
        tbe.tbe_set_forward_scratch(h, buf, need)
        tbe.tbe_forward(h, spec.B, pb.idx, pb.off, None, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        # contents need no initialisation: garbage in the scratch, same bits
        buf.fill_(0xAB)
        tbe.tbe_forward(h, spec.B, pb.idx, pb.off, None, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        tbe.tbe_set_forward_scratch(h, None, 0)                                # detach
        assert _status(tbe.tbe_forward, h, spec.B, pb.idx, pb.off, None, out) == 4
    finally:
        tbe.tbe_destroy(h)
        pb.op.close()


def test_handles_without_opt_in_paths_need_no_scratch():
    spec = workloads.config(1)
    pb = make_problem(spec, seed=4)
    h = _raw_handle(spec, pb.W, 0)
    try:
        assert tbe.tbe_forward_scratch_size(h) == 0
        out = torch.empty((spec.B, sum(spec.dims)), dtype=torch.float32, device="cuda")
        tbe.tbe_forward(h, spec.B, pb.idx, pb.off, None, out)
        torch.cuda.synchronize()
        assert torch.equal(out, pb.op.forward(spec.B, pb.idx, pb.off))
    finally:
        tbe.tbe_destroy(h)
        pb.op.close()
