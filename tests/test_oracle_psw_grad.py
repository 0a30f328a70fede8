"""Pins of the oracle's gradient with respect to the per-sample weights.

The forward takes per-sample weights (kimbodo.com/?p=28372, "What Happened") and is linear in
them: Y[b, doff_t + d] = s_k * sum_i p_i * W_t[x_i, d].  Hence
dL/dp_i = s_k * <G[b, doff_t : doff_t + D_t], W_t[x_i]> for L = <G, Y>.

Pins: torch autograd through embedding_bag in float64 (library), exact finite differences of
<G, forward(p)> (the forward is linear in p, so only fp64 rounding remains), the mean-pooling scale,
and an empty batch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _np_weights(spec, seed=0):
    return workloads.storage_numpy(workloads.weights(spec, seed)).copy()


def _np_grad(spec, seed=0):
    return workloads.grad_output(spec, seed, 0).numpy()


def _layout(spec):
    dims = np.array(spec.dims, np.int64)
    rows = np.array(spec.rows, np.int64)
    woff = np.concatenate([[0], np.cumsum(rows * dims)])
    doff = np.concatenate([[0], np.cumsum(dims)])
    return rows, dims, woff, doff


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_matches_torch_autograd(dtype):
    """Sum pooling: per table, torch embedding_bag (float64) with per_sample_weights, then
    autograd of <G, Y> with respect to the weights."""
    spec = workloads.custom([50, 7, 300], [8, 16, 32], dtype, B=21, lengths=("uniform_int", 0, 9),
                            psw=True, key=401)
    batch = workloads.batch(spec, 0, 0)
    W = _np_weights(spec)
    G = _np_grad(spec)
    got = oracle.psw_grad(spec.rows, spec.dims, workloads.oracle_dtype(dtype), oracle.POOL_SUM, W,
                          spec.B, batch.indices, batch.offsets, G)
    Wd = oracle.widen(workloads.oracle_dtype(dtype), W)
    rows, dims, woff, doff = _layout(spec)
    for t in range(spec.T):
        table = torch.from_numpy(Wd[woff[t]:woff[t + 1]].reshape(rows[t], dims[t]))
        o = batch.offsets[t * spec.B:(t + 1) * spec.B + 1]
        lo, hi = int(o[0]), int(o[-1])
        ids = torch.from_numpy(batch.indices[lo:hi])
        p = torch.from_numpy(batch.psw[lo:hi].astype(np.float64)).requires_grad_(True)
        offs = torch.from_numpy(o[:-1] - lo)
        Y = torch.nn.functional.embedding_bag(ids, table, offs, mode="sum", per_sample_weights=p)
        g = torch.from_numpy(G[:, doff[t]:doff[t + 1]].astype(np.float64))
        (Y * g).sum().backward()
        np.testing.assert_allclose(got[lo:hi], p.grad.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("pooling", [oracle.POOL_SUM, oracle.POOL_MEAN])
def test_exact_finite_differences(pooling):
    """<G, Y(p + h e_i)> - <G, Y(p)> = h * dL/dp_i up to fp64 rounding (linear in p), with h
    the fp32 step actually taken."""
    spec = workloads.custom([40, 13], [4, 12], "f32", B=9, lengths=("uniform_int", 0, 7), psw=True,
                            pooling="mean" if pooling == oracle.POOL_MEAN else "sum", key=402)
    batch = workloads.batch(spec, 0, 0)
    W = _np_weights(spec)
    G = _np_grad(spec).astype(np.float64)
    got = oracle.psw_grad(spec.rows, spec.dims, oracle.F32, pooling, W, spec.B, batch.indices,
                          batch.offsets, G.astype(np.float32))
    G32 = G.astype(np.float32).astype(np.float64)

    def loss(p):
        Y = oracle.forward(spec.rows, spec.dims, oracle.F32, pooling, W, spec.B, batch.indices,
                           batch.offsets, p)
        return float((Y * G32).sum())

    base = loss(batch.psw)
    rng = np.random.default_rng(5)
    for i in rng.choice(batch.N, size=min(25, batch.N), replace=False):
        p = batch.psw.copy()
        p[i] += np.float32(0.25)
        h = float(p[i]) - float(batch.psw[i])  # the step actually taken (fp32 rounding)
        fd = (loss(p) - base) / h
        assert abs(fd - got[i]) <= 1e-9 * (1.0 + abs(got[i])), (i, fd, got[i])


def test_mean_scale():
    """Mean pooling divides each lookup's gradient by its bag's length (not by sum p)."""
    spec = workloads.custom([60], [16], "bf16", B=15, lengths=("uniform_int", 1, 12), psw=True,
                            key=403)
    batch = workloads.batch(spec, 0, 0)
    W = _np_weights(spec)
    G = _np_grad(spec)
    s = oracle.psw_grad(spec.rows, spec.dims, oracle.BF16, oracle.POOL_SUM, W, spec.B,
                        batch.indices, batch.offsets, G)
    m = oracle.psw_grad(spec.rows, spec.dims, oracle.BF16, oracle.POOL_MEAN, W, spec.B,
                        batch.indices, batch.offsets, G)
    lens = np.repeat(np.diff(batch.offsets), np.diff(batch.offsets))
    np.testing.assert_allclose(m, s / lens, rtol=1e-15)


def test_empty_batch():
    spec = workloads.custom([10], [4], "f32", B=3, lengths=("fixed", 0), psw=True, key=404)
    batch = workloads.batch(spec, 0, 0)
    out = oracle.psw_grad(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, _np_weights(spec),
                          spec.B, batch.indices, batch.offsets, _np_grad(spec))
    assert out.size == 0
