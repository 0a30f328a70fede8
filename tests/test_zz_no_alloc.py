"""tbe_backward_update_no_alloc, the backward for callers that cannot allocate: the same
kernels as tbe_backward_update on a static device array inside the library instead of a
caller workspace.  Checked against tbe_backward_update on a second handle with identical
weights and state: runs, weights and state bit-identical, over two calls in a row on the
shared array, the second with a smaller batch (the array then holds the first call's
contents)."""
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import check_runs, gpu_runs, make_problem, to_device

pytestmark = pytest.mark.gpu

BIG = workloads.config(2)   # 8 tables of 100k x 128 fp32, 270k Zipf(1.05) lookups, Adagrad


def _smaller(spec, B, key):
    return workloads.custom(spec.rows, spec.dims, spec.dtype, B=B, lengths=spec.lengths,
                            index_dist=spec.index_dist, pooling=spec.pooling, psw=spec.psw,
                            optimizer=spec.optimizer, key=key)


CASES = {
    "270k-f32-adagrad": (BIG, _smaller(BIG, 300, 601)),
    "bf16-mean-psw-mixed-dims": (
        workloads.custom([5000, 700, 90], [64, 32, 8], "bf16", B=4000,
                         lengths=("uniform_int", 0, 40), index_dist=("zipf", 1.2),
                         pooling="mean", psw=True, optimizer="rowwise_adagrad", key=602),
        workloads.custom([5000, 700, 90], [64, 32, 8], "bf16", B=37,
                         lengths=("uniform_int", 0, 40), index_dist=("zipf", 1.2),
                         pooling="mean", psw=True, optimizer="rowwise_adagrad", key=603)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_no_alloc_backward_equals_the_workspace_backward(case):
    first, second = CASES[case]
    print(f"[no-alloc] {case}", flush=True)
    a = make_problem(first, seed=5)     # tbe_backward_update, caller workspace
    b = make_problem(first, seed=5)     # tbe_backward_update_no_alloc, static scratch
    for step, spec in enumerate((first, second)):
        batch = workloads.batch(spec, seed=5, step=step)
        need = tbe.tbe_backward_workspace_size(b.op.handle, spec.B, batch.N)
        assert need <= tbe.STATIC_SCRATCH_BYTES
        idx, off, psw = to_device(batch)
        G = workloads.grad_output(spec, seed=5, step=step, device="cuda")
        ra, rb = gpu_runs(a, batch.N), gpu_runs(b, batch.N)
        a.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps, ra)
        tbe.tbe_backward_update_no_alloc(b.op.handle, spec.B, idx, off, psw, G, spec.lr,
                                         spec.eps, rb)
        torch.cuda.synchronize()
        U = int(ra[2].item())
        assert int(rb[2].item()) == U
        assert torch.equal(ra[0][:U], rb[0][:U]) and torch.equal(ra[1][:U], rb[1][:U])
        b.spec, b.batch = spec, batch
        check_runs(b, rb)                  # and the grouping is the reference's
        assert torch.equal(a.W, b.W), f"call {step}: weights"
        assert torch.equal(a.state, b.state), f"call {step}: state"
        a.check_guards()
        b.check_guards()
        print(f"  call {step}: {batch.N} lookups, identical", flush=True)
    b.op.check_device_status()
    a.op.close()
    b.op.close()


def test_no_alloc_backward_rejects_a_batch_larger_than_its_scratch():
    spec = workloads.custom([100_000] * 2, [128, 128], "f32", B=65536, lengths=("fixed", 16),
                            key=604)
    n = 2 * 65536 * 16
    pb = make_problem(workloads.custom([100_000] * 2, [128, 128], "f32", B=4, key=605), seed=0)
    assert tbe.tbe_backward_workspace_size(pb.op.handle, spec.B, n) > tbe.STATIC_SCRATCH_BYTES
    idx = torch.zeros(n, dtype=torch.int64, device="cuda")
    off = torch.zeros(2 * spec.B + 1, dtype=torch.int64, device="cuda")
    G = torch.zeros((spec.B, 256), device="cuda")
    W0 = pb.W.clone()
    with pytest.raises(tbe.TBEError, match="WORKSPACE_TOO_SMALL"):
        tbe.tbe_backward_update_no_alloc(pb.op.handle, spec.B, idx, off, None, G, 0.1, 1e-8)
    torch.cuda.synchronize()
    assert torch.equal(pb.W, W0)
    pb.op.close()
