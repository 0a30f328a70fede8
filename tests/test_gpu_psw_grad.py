"""GPU parity of the per-sample-weight gradient (tbe_psw_grad) against the CPU reference.

dL/dp_i = s_k * <G[b, doff_t : doff_t + D_t], W_t[x_i]>: the forward takes per-sample weights
(kimbodo.com/?p=28372, "What Happened") and is linear in them.  Tolerance: the fp32 dot
product of D terms is within 1e-5 * s_k * sum_d |G_d W_d| of the exact value (well above the
bound D * 2^-24 for D <= 1024).
"""
import numpy as np
import pytest
import torch

import oracle
import table_embedding_bag_amd as tbe
import workloads
from gpu_check import abs_bits, code, make_problem, pool, to_device
from test_gpu_parity import UNIT

pytestmark = pytest.mark.gpu


def _check(spec, seed=0, index_dtype=torch.int64, batch=None):
    pb = make_problem(spec, seed=seed, index_dtype=index_dtype, batch=batch)
    G = workloads.grad_output(spec, seed=seed, step=0, device="cuda")
    got = pb.op.psw_grad(spec.B, pb.idx, pb.off, G)
    torch.cuda.synchronize()
    W = workloads.storage_numpy(pb.W)
    Gh = G.cpu().numpy()
    ref = oracle.psw_grad(spec.rows, spec.dims, code(spec), pool(spec), W, spec.B,
                          pb.batch.indices, pb.batch.offsets, Gh)
    scale = oracle.psw_grad(spec.rows, spec.dims, code(spec), pool(spec), abs_bits(spec, W),
                            spec.B, pb.batch.indices, pb.batch.offsets, np.abs(Gh))
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    bad = err > 1e-5 * scale + 1e-30
    assert not bad.any(), (f"{bad.sum()} of {bad.size} lookups off; worst "
                           f"{(err / np.maximum(scale, 1e-30)).max():.2e} of sum |G W|")
    pb.op.close()


@pytest.mark.parametrize("spec", [UNIT[0], UNIT[2], UNIT[3], UNIT[4], UNIT[5], UNIT[6], UNIT[7],
                                  UNIT[8], UNIT[10]],
                         ids=lambda s: f"{s.key}-{s.dtype}-{s.pooling}-psw{int(s.psw)}")
def test_psw_grad_parity(spec):
    _check(spec, seed=21)


def test_psw_grad_int32_indices():
    _check(UNIT[4], seed=22, index_dtype=torch.int32)


@pytest.mark.timeout(600)
def test_psw_grad_32_mixed_bf16_tables():
    """Mixed dims 32..256, bf16, mean pooling with weights: the workload that trains them."""
    _check(workloads.config(3), seed=0)


def test_psw_grad_empty_bags():
    spec = workloads.custom([30, 9], [16, 8], "f32", B=6, psw=True, key=408)
    lens = [0, 3, 0, 0, 5, 1, 2, 0, 0, 0, 4, 0]
    rng = np.random.default_rng(3)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = np.concatenate([rng.integers(0, spec.rows[k // spec.B], size=lens[k])
                          for k in range(len(lens))]).astype(np.int64)
    batch = workloads.Batch(idx, off, rng.random(idx.size).astype(np.float32))
    _check(spec, seed=23, batch=batch)
