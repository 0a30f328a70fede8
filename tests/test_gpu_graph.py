"""The training step captured in a HIP graph.  Without TBE_FLAG_VALIDATE and profiling, the
calls queue kernels only (no host synchronisation, no allocation, no memset nodes), so the
pair tbe_forward_group + tbe_backward_update_grouped (and tbe_forward + tbe_backward_update)
can be captured once per batch and replayed.  Each replay must give the same output, weights
and state as the same calls made eagerly, bit for bit.  The replays are checked one by one,
with eager work and synchronisations between them."""
import pytest
import torch

import workloads
from gpu_check import make_problem, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _pair(pb, spec, idx, off, psw, G, Y, grouped):
    if grouped:
        pb.op.forward_group(spec.B, idx, off, psw, out=Y)
        pb.op.backward_update_grouped(spec.B, idx, off, psw, G, spec.lr, spec.eps)
    else:
        pb.op.forward(spec.B, idx, off, psw, out=Y)
        pb.op.backward_update(spec.B, idx, off, psw, G, spec.lr, spec.eps)


@pytest.mark.parametrize("grouped", [True, False], ids=["grouped", "plain"])
@pytest.mark.parametrize("n", [2, 3], ids=["270k-lookups", "5.2M-lookups"])
def test_graph_replays_match_eager_calls(n, grouped):
    spec = workloads.config(n)
    _say(f"[graph] workload {n} grouped={grouped}")
    a = make_problem(spec, seed=31)   # eager
    b = make_problem(spec, seed=31)   # captured
    batches = [to_device(workloads.batch(spec, seed=31, step=s)) for s in range(2)]
    grads = [workloads.grad_output(spec, seed=31, step=s, device="cuda") for s in range(2)]
    Ya = torch.empty((spec.B, sum(spec.dims)), dtype=torch.float32, device="cuda")
    Yb = torch.empty_like(Ya)
    # one eager pair on b first (its workspace is allocated outside the capture), then undo
    # its update by restoring b's weights and state from a
    _pair(b, spec, *batches[0], grads[0], Yb, grouped)
    torch.cuda.synchronize()
    b.W.copy_(a.W)
    if b.state is not None:
        b.state.copy_(a.state)
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                _pair(b, spec, *batches[s], grads[s], Yb, grouped)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capturing ran nothing: b is still at the starting point
    assert torch.equal(b.W, a.W)
    for step in range(5):
        s = step % 2
        _pair(a, spec, *batches[s], grads[s], Ya, grouped)
        graphs[s].replay()
        torch.cuda.synchronize()
        assert torch.equal(Ya, Yb), f"step {step}: output"
        assert torch.equal(a.W, b.W), f"step {step}: weights"
        if a.state is not None:
            assert torch.equal(a.state, b.state), f"step {step}: state"
        # eager work on the stream between replays
        Ya.mul_(1.0)
        _say(f"  replay {step}: identical")
    a.op.close()
    b.op.close()
