"""Pins of the oracle's pooled forward.

The forward gathers the rows a bag selects and aggregates them into one dense
vector per sample and table ("FBTriton Rewrites Table Batched Embedding",
"Responsibilities of the forward and backward passes"), over all tables at
once, optionally scaled by per-sample weights (kimbodo.com/?p=28372, "What
Happened").  The batch is a flat id list plus CSR offsets ("Optimizing
Recommendation Systems with FBTriton Table Batched Embeddings", "Implementation
Guide: Integrating TBE").

Pins: the page's worked example (structure), torch's CPU embedding_bag in
fp64 (library routine), a dense count-matrix product (brute force), linearity,
and the special cases (empty bag, mean with weights).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dyadic_table(E, D):
    # exactly representable values so sums are exact in any order
    r = np.arange(E, dtype=np.float64)[:, None]
    d = np.arange(D, dtype=np.float64)[None, :]
    return (r + d / 4.0).astype(np.float32)


def test_worked_example_bags():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    E, D = 16, 4
    W = _dyadic_table(E, D)
    idx = np.array(ex["indices"], dtype=np.int64)
    off = np.array(ex["offsets"], dtype=np.int64)
    B = len(off) - 1  # one table
    Y = oracle.forward([E], [D], oracle.F32, oracle.POOL_SUM, W.reshape(-1), B, idx, off)
    assert Y.shape == (len(ex["bags"]), D)
    for b, bag in enumerate(ex["bags"]):
        assert np.array_equal(Y[b], W[bag].astype(np.float64).sum(axis=0))


def _per_table_torch(spec, W64, batch, mode):
    """torch.nn.functional.embedding_bag per table, fp64 CPU."""
    outs = []
    woff = 0
    for t in range(spec.T):
        E, D = spec.rows[t], spec.dims[t]
        table = torch.from_numpy(W64[woff:woff + E * D].reshape(E, D))
        woff += E * D
        lo, hi = batch.offsets[t * spec.B], batch.offsets[(t + 1) * spec.B]
        idx = torch.from_numpy(batch.indices[lo:hi])
        off = torch.from_numpy(batch.offsets[t * spec.B:(t + 1) * spec.B + 1] - lo)
        psw = None
        if batch.psw is not None:
            psw = torch.from_numpy(batch.psw[lo:hi].astype(np.float64))
        outs.append(torch.nn.functional.embedding_bag(idx, table, off, mode=mode,
                                                      per_sample_weights=psw,
                                                      include_last_offset=True).numpy())
    return np.concatenate(outs, axis=1)


def _weights_np(spec, seed=0):
    w = workloads.weights(spec, seed)
    return workloads.storage_numpy(w)


def _run_oracle(spec, W, batch):
    return oracle.forward(spec.rows, spec.dims, workloads.oracle_dtype(spec.dtype),
                          oracle.POOL_MEAN if spec.pooling == "mean" else oracle.POOL_SUM,
                          W, spec.B, batch.indices, batch.offsets, batch.psw)


CASES = [
    workloads.config(1),
    workloads.custom([50, 7, 300], [8, 3, 16], "f32", B=11, lengths=("uniform_int", 0, 9)),
    workloads.custom([50, 7, 300], [8, 3, 16], "bf16", B=11, lengths=("uniform_int", 0, 9)),
    workloads.custom([20, 90], [32, 5], "f16", B=9, lengths=("uniform_int", 0, 12),
                     index_dist=("zipf", 1.2)),
    workloads.custom([20, 90], [32, 5], "f32", B=9, lengths=("uniform_int", 0, 12), pooling="mean"),
    workloads.custom([20, 90], [32, 5], "bf16", B=9, lengths=("uniform_int", 0, 12), pooling="mean"),
    workloads.custom([40, 13, 9], [4, 12, 64], "f32", B=10, lengths=("uniform_int", 0, 8), psw=True),
    workloads.custom([40, 13, 9], [4, 12, 64], "f16", B=10, lengths=("uniform_int", 0, 8), psw=True),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: f"{s.name}-{s.dtype}-{s.pooling}-psw{int(s.psw)}")
def test_forward_matches_torch_embedding_bag(spec):
    batch = workloads.batch(spec, seed=0)
    W = _weights_np(spec)
    W64 = oracle.widen(workloads.oracle_dtype(spec.dtype), W)
    ref = _per_table_torch(spec, W64, batch, spec.pooling)
    got = _run_oracle(spec, W, batch)
    scale = np.abs(ref).max() + 1e-300
    assert np.abs(got - ref).max() <= 1e-12 * scale


def _dense_count_matrix(spec, batch):
    """A[k, r] = sum over lookups of bag k hitting linear row r of p_i * s_k."""
    nb = spec.T * spec.B
    A = np.zeros((nb, spec.sum_rows))
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    for k in range(nb):
        t = k // spec.B
        lo, hi = batch.offsets[k], batch.offsets[k + 1]
        for i in range(lo, hi):
            p = 1.0 if batch.psw is None else float(batch.psw[i])
            if spec.pooling == "mean":
                p /= (hi - lo)
            A[k, roff[t] + batch.indices[i]] += p
    return A


def _block_diag_weights(spec, W64):
    """The stacked tables as one [sum E, sum D] block-diagonal matrix."""
    M = np.zeros((spec.sum_rows, spec.sum_dims))
    r = c = w = 0
    for t in range(spec.T):
        E, D = spec.rows[t], spec.dims[t]
        M[r:r + E, c:c + D] = W64[w:w + E * D].reshape(E, D)
        r, c, w = r + E, c + D, w + E * D
    return M


BRUTE = [
    workloads.custom([12, 5], [3, 6], "f32", B=7, lengths=("uniform_int", 0, 6), pooling="mean", psw=True),
    workloads.custom([12, 5], [3, 6], "bf16", B=7, lengths=("uniform_int", 0, 6), pooling="sum", psw=True),
    workloads.custom([9], [4], "f16", B=5, lengths=("uniform_int", 0, 10), pooling="mean"),
]


@pytest.mark.parametrize("spec", BRUTE, ids=lambda s: f"{s.dtype}-{s.pooling}-psw{int(s.psw)}")
def test_forward_equals_dense_count_matrix_product(spec):
    batch = workloads.batch(spec, seed=4)
    W = _weights_np(spec, seed=4)
    W64 = oracle.widen(workloads.oracle_dtype(spec.dtype), W)
    A = _dense_count_matrix(spec, batch)
    M = _block_diag_weights(spec, W64)
    full = A @ M  # [T*B, sum D]; row k holds bag k in its table's columns
    got = _run_oracle(spec, W, batch)
    doff = np.concatenate([[0], np.cumsum(spec.dims)])
    for t in range(spec.T):
        ref = full[t * spec.B:(t + 1) * spec.B, doff[t]:doff[t + 1]]
        assert np.abs(got[:, doff[t]:doff[t + 1]] - ref).max() <= 1e-12 * (np.abs(ref).max() + 1e-300)


def test_forward_linearity_in_weights_and_psw():
    spec = workloads.custom([30, 17], [8, 5], "f32", B=6, lengths=("uniform_int", 0, 7), psw=True)
    batch = workloads.batch(spec, seed=2)
    rng = np.random.default_rng(2)
    # small integers: all sums exact in fp64, all values exact in fp32
    W1 = rng.integers(-64, 64, spec.num_weights).astype(np.float32)
    W2 = rng.integers(-64, 64, spec.num_weights).astype(np.float32)
    a, b = 3.0, -2.0
    f = lambda W, p: oracle.forward(spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM, W, spec.B,
                                    batch.indices, batch.offsets, p)
    p = rng.integers(0, 4, batch.N).astype(np.float32)
    assert np.array_equal(f((a * W1 + b * W2).astype(np.float32), p), a * f(W1, p) + b * f(W2, p))
    q = rng.integers(0, 4, batch.N).astype(np.float32)
    assert np.array_equal(f(W1, p + q), f(W1, p) + f(W1, q))
    # splitting a bag into two bags splits its sum
    idx = batch.indices[batch.offsets[0]:batch.offsets[spec.B]]
    n0 = idx.size
    s = n0 // 2
    whole = oracle.forward([30], [8], oracle.F32, oracle.POOL_SUM, W1[:240], 1, idx,
                           np.array([0, n0], dtype=np.int64))
    parts = oracle.forward([30], [8], oracle.F32, oracle.POOL_SUM, W1[:240], 2, idx,
                           np.array([0, s, n0], dtype=np.int64))
    assert np.array_equal(whole[0], parts[0] + parts[1])


def test_mean_of_empty_bag_is_zero_and_mean_with_psw_is_weighted_sum_over_length():
    E, D = 10, 4
    W = np.random.default_rng(0).standard_normal(E * D).astype(np.float32)
    idx = np.array([1, 2, 3, 3, 9], dtype=np.int64)
    off = np.array([0, 0, 2, 5], dtype=np.int64)  # bag 0 empty
    psw = np.array([0.5, 2.0, 1.0, 0.25, 3.0], dtype=np.float32)
    mean = oracle.forward([E], [D], oracle.F32, oracle.POOL_MEAN, W, 3, idx, off, psw)
    wsum = oracle.forward([E], [D], oracle.F32, oracle.POOL_SUM, W, 3, idx, off, psw)
    assert np.array_equal(mean[0], np.zeros(D)) and not np.isnan(mean).any()
    lens = np.diff(off)
    for b in (1, 2):
        assert np.allclose(mean[b], wsum[b] / lens[b], rtol=1e-15, atol=0)
    # with all weights 1, mean+weights reduces to torch's plain mean
    ones = np.ones_like(psw)
    m1 = oracle.forward([E], [D], oracle.F32, oracle.POOL_MEAN, W, 3, idx, off, ones)
    ref = torch.nn.functional.embedding_bag(torch.from_numpy(idx), torch.from_numpy(W.astype(np.float64)).view(E, D),
                                            torch.from_numpy(off), mode="mean",
                                            include_last_offset=True).numpy()
    assert np.allclose(m1, ref, rtol=1e-15, atol=0)


def test_single_lookup_returns_stored_row_exactly():
    for dt in (oracle.F16, oracle.BF16):
        bits = np.random.default_rng(1).integers(0, 0x7C00, size=5 * 8).astype(np.uint16)
        idx = np.array([3], dtype=np.int64)
        Y = oracle.forward([5], [8], dt, oracle.POOL_SUM, bits, 1, idx, np.array([0, 1], np.int64))
        assert np.array_equal(Y[0], oracle.widen(dt, bits[24:32]))


def test_forward_bags_subset_matches_full():
    spec = CASES[6]
    batch = workloads.batch(spec, seed=0)
    W = _weights_np(spec)
    full = _run_oracle(spec, W, batch)
    ids = np.array([0, 5, 12, 29, 17], dtype=np.int64)
    parts = oracle.forward_bags(spec.rows, spec.dims, 0, 0, W, spec.B, batch.indices, batch.offsets,
                                batch.psw, ids)
    doff = np.concatenate([[0], np.cumsum(spec.dims)])
    for k, v in zip(ids, parts):
        t, b = divmod(int(k), spec.B)
        assert np.array_equal(v, full[b, doff[t]:doff[t + 1]])


@pytest.mark.parametrize("bad", ["index_high", "index_negative", "offsets_total", "offsets_decreasing"])
def test_invalid_batches_are_rejected(bad):
    idx = np.array([1, 2, 3], dtype=np.int64)
    off = np.array([0, 1, 3], dtype=np.int64)
    if bad == "index_high":
        idx[1] = 10
    elif bad == "index_negative":
        idx[0] = -1
    elif bad == "offsets_total":
        off[-1] = 2
    else:
        off[1] = 4
    W = np.zeros(40, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.forward([10], [4], oracle.F32, oracle.POOL_SUM, W, 2, idx, off)


def test_timing_build_agrees_with_the_reference_to_fp32_rounding(tmp_path):
    """The CPU-baseline build (same source, fp32 accumulators) computes the same thing:
    its forward and its update agree with the fp64 reference to fp32 rounding.  It is only
    ever timed; parity always uses the fp64 build."""
    lib = oracle.load_timed(oracle.build_timed(str(tmp_path / "libtbe_oracle_f32.so")))
    spec = workloads.custom([300, 41], [16, 8], "f32", B=64, lengths=("uniform_int", 0, 20),
                            index_dist=("zipf", 1.2), optimizer="rowwise_adagrad", psw=True)
    batch = workloads.batch(spec, seed=3)
    W = workloads.storage_numpy(workloads.weights(spec, 3)).copy()
    G = workloads.grad_output(spec, 3).numpy()
    args = (spec.rows, spec.dims, oracle.F32, oracle.POOL_SUM)
    Y64 = oracle.forward(*args, W, spec.B, batch.indices, batch.offsets, batch.psw)
    Y32 = oracle.forward(*args, W, spec.B, batch.indices, batch.offsets, batch.psw, lib=lib)
    scale = oracle.forward(*args, np.abs(W), spec.B, batch.indices, batch.offsets, np.abs(batch.psw))
    assert (np.abs(Y32 - Y64) <= 1e-5 * scale + 1e-30).all()
    W64, W32 = W.copy(), W.copy()
    s64, s32 = np.zeros(spec.sum_rows, np.float32), np.zeros(spec.sum_rows, np.float32)
    for Wx, sx, lb in ((W64, s64, None), (W32, s32, lib)):
        oracle.backward_update(*args, oracle.OPT_ROWWISE_ADAGRAD, Wx, sx, spec.B, batch.indices,
                               batch.offsets, batch.psw, G, 0.01, 1e-8, lib=lb)
    assert np.allclose(s32, s64, rtol=1e-5, atol=0)
    assert np.all(np.abs(W32 - W64) <= 1e-5 * (np.abs(W) + 0.01))
