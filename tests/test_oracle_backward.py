"""Pins of the oracle's grouping and its one-update-per-row backward.

The backward scatters upstream gradients back to the looked-up rows and adds
them up where a row was hit more than once ("FBTriton Rewrites Table Batched
Embedding", "Responsibilities of the forward and backward passes"); updates are
grouped by (table, row) so that every touched row gets one optimizer update
(kimbodo.com/?p=28372, "What Happened"), via a transpose, sort and run-length
encoding ("Kimbodo Engineering Perspective").  The pages name no optimizer:
plain SGD and row-wise Adagrad are readings, pinned here by their closed forms.

Pins: numpy unique / bincount (library), the dense transpose product A^T G
(brute force), central finite differences of <G, forward(W)>, the duplicate
invariant, closed forms of both optimizers, untouched rows, and
torch.optim.Adagrad on one-column tables (where row-wise Adagrad is plain
Adagrad), which fixes the update order and where eps sits.  The mean over the
row for wider rows stays a reading.
"""
import numpy as np
import pytest

import oracle
import workloads

LR = float(np.float32(0.01))
EPS = float(np.float32(1e-8))


def _np_weights(spec, seed=0):
    return workloads.storage_numpy(workloads.weights(spec, seed)).copy()


def _np_grad(spec, seed=0, step=0):
    return workloads.grad_output(spec, seed, step).numpy()


def _pool(spec):
    return oracle.POOL_MEAN if spec.pooling == "mean" else oracle.POOL_SUM


def _opt(spec):
    return oracle.OPT_ROWWISE_ADAGRAD if spec.optimizer == "rowwise_adagrad" else oracle.OPT_SGD


def _linear_ids(spec, batch):
    # table of each lookup from the bag it sits in, then table row offset + row
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    bag = np.repeat(np.arange(spec.T * spec.B), np.diff(batch.offsets))
    return roff[bag // spec.B] + batch.indices


SPECS = [
    workloads.config(1),
    workloads.custom([300, 41, 7], [8, 3, 16], "f32", B=40, lengths=("uniform_int", 0, 20),
                     index_dist=("zipf", 1.3)),
    workloads.custom([5000, 64], [4, 4], "f32", B=512, lengths=("fixed", 16), index_dist=("zipf", 1.5)),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_runs_match_numpy_unique_and_bincount(spec):
    batch = workloads.batch(spec, seed=1)
    uniq, cnt = oracle.runs(spec.rows, spec.B, batch.indices, batch.offsets)
    ref_u, ref_c = np.unique(_linear_ids(spec, batch), return_counts=True)
    assert np.array_equal(uniq, ref_u) and np.array_equal(cnt, ref_c)
    # per table: bincount of the table-local ids gives the same counts
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    for t in range(spec.T):
        lo, hi = batch.offsets[t * spec.B], batch.offsets[(t + 1) * spec.B]
        bc = np.bincount(batch.indices[lo:hi], minlength=spec.rows[t])
        sel = (uniq >= roff[t]) & (uniq < roff[t + 1])
        assert np.array_equal(np.nonzero(bc)[0], uniq[sel] - roff[t])
        assert np.array_equal(bc[bc > 0], cnt[sel])


def test_runs_of_empty_batch():
    off = np.zeros(2 * 3 + 1, dtype=np.int64)
    u, c = oracle.runs([10, 10], 3, np.zeros(0, np.int64), off)
    assert u.size == 0 and c.size == 0


def _dense_AtG(spec, batch, G):
    """Brute force: Gamma = A^T G with A the per-bag count matrix (weights, mean scale)."""
    doff = np.concatenate([[0], np.cumsum(spec.dims)])
    woff = np.concatenate([[0], np.cumsum(np.array(spec.rows) * np.array(spec.dims))])
    out = np.zeros(spec.num_weights)
    for t in range(spec.T):
        E, D = spec.rows[t], spec.dims[t]
        A = np.zeros((spec.B, E))
        for b in range(spec.B):
            k = t * spec.B + b
            lo, hi = batch.offsets[k], batch.offsets[k + 1]
            for i in range(lo, hi):
                p = 1.0 if batch.psw is None else float(batch.psw[i])
                if spec.pooling == "mean":
                    p /= (hi - lo)
                A[b, batch.indices[i]] += p
        out[woff[t]:woff[t + 1]] = (A.T @ G[:, doff[t]:doff[t + 1]].astype(np.float64)).reshape(-1)
    return out


GRAD_SPECS = [
    workloads.custom([30, 9], [5, 8], "f32", B=12, lengths=("uniform_int", 0, 9), pooling="mean", psw=True),
    workloads.custom([30, 9], [5, 8], "f32", B=12, lengths=("uniform_int", 0, 9), index_dist=("zipf", 1.4)),
    workloads.custom([7], [3], "f32", B=20, lengths=("uniform_int", 0, 5), pooling="mean"),
]


@pytest.mark.parametrize("spec", GRAD_SPECS, ids=lambda s: f"{s.pooling}-psw{int(s.psw)}-{s.index_dist[0]}")
def test_dense_grad_equals_transpose_product(spec):
    batch = workloads.batch(spec, seed=3)
    G = _np_grad(spec, seed=3)
    got = oracle.dense_grad(spec.rows, spec.dims, _pool(spec), spec.B, batch.indices, batch.offsets,
                            batch.psw, G)
    ref = _dense_AtG(spec, batch, G)
    assert np.abs(got - ref).max() <= 1e-12 * (np.abs(ref).max() + 1e-300)


def test_dense_grad_equals_finite_differences_of_forward():
    # l(W) = <G, forward(W)> is linear in W, so a central difference with a
    # power-of-two step on dyadic weights is exact up to fp64 rounding.
    spec = workloads.custom([11, 6], [4, 3], "f32", B=9, lengths=("uniform_int", 0, 7),
                            pooling="mean", psw=True)
    batch = workloads.batch(spec, seed=5)
    G = _np_grad(spec, seed=5)
    rng = np.random.default_rng(5)
    W = (rng.integers(-512, 512, spec.num_weights) / 256.0).astype(np.float32)
    grad = oracle.dense_grad(spec.rows, spec.dims, oracle.POOL_MEAN, spec.B, batch.indices,
                             batch.offsets, batch.psw, G)

    def loss(Wx):
        Y = oracle.forward(spec.rows, spec.dims, oracle.F32, oracle.POOL_MEAN, Wx, spec.B,
                           batch.indices, batch.offsets, batch.psw)
        return float((Y * G.astype(np.float64)).sum())

    h = 0.5
    fd = np.empty(spec.num_weights)
    for j in range(spec.num_weights):
        Wp, Wm = W.copy(), W.copy()
        Wp[j] += h
        Wm[j] -= h
        fd[j] = (loss(Wp) - loss(Wm)) / (2 * h)
    assert np.abs(fd - grad).max() <= 1e-10 * (np.abs(grad).max() + 1e-300)


def _update(spec, W, state, batch, G, selected=None):
    oracle.backward_update(spec.rows, spec.dims, workloads.oracle_dtype(spec.dtype), _pool(spec),
                           _opt(spec), W, state, spec.B, batch.indices, batch.offsets, batch.psw, G,
                           spec.lr, spec.eps, selected)


@pytest.mark.parametrize("pooling,psw", [("sum", False), ("mean", True)])
def test_sgd_step_is_minus_lr_times_summed_gradient(pooling, psw):
    spec = workloads.custom([40, 13], [8, 5], "f32", B=16, lengths=("uniform_int", 0, 9),
                            pooling=pooling, psw=psw, index_dist=("zipf", 1.2), lr=LR)
    batch = workloads.batch(spec, seed=6)
    G = _np_grad(spec, seed=6)
    W0 = _np_weights(spec, seed=6)
    W = W0.copy()
    _update(spec, W, None, batch, G)
    ref = W0.astype(np.float64) - LR * _dense_AtG(spec, batch, G)
    # one rounding to fp32 of the exact fp64 value
    assert np.array_equal(W, ref.astype(np.float32))


def test_untouched_rows_are_bit_identical():
    spec = workloads.custom([200, 50], [6, 4], "bf16", B=8, lengths=("uniform_int", 0, 4),
                            optimizer="rowwise_adagrad")
    batch = workloads.batch(spec, seed=8)
    G = _np_grad(spec, seed=8)
    W0 = _np_weights(spec, seed=8)
    W = W0.copy()
    st = np.zeros(spec.sum_rows, np.float32)
    _update(spec, W, st, batch, G)
    touched = np.zeros(spec.sum_rows, bool)
    touched[_linear_ids(spec, batch)] = True
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    woff = np.concatenate([[0], np.cumsum(np.array(spec.rows) * np.array(spec.dims))])
    for t in range(spec.T):
        D = spec.dims[t]
        w0 = W0[woff[t]:woff[t + 1]].reshape(-1, D)
        w1 = W[woff[t]:woff[t + 1]].reshape(-1, D)
        tt = touched[roff[t]:roff[t + 1]]
        assert np.array_equal(w0[~tt], w1[~tt])
        assert (w0[tt] != w1[tt]).any(axis=1).all()
    assert (st[~touched] == 0).all() and (st[touched] > 0).all()


@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
def test_duplicates_equal_one_lookup_with_summed_gradient(optimizer):
    # row 3 of a one-table problem hit k times with gradients g_1..g_k (dyadic)
    # must give bit-identical weights and state to one hit with g_1+...+g_k.
    E, D, k = 8, 4, 5
    spec = workloads.custom([E], [D], "f32", B=k, optimizer=optimizer, lr=0.25, eps=0.0)
    rng = np.random.default_rng(9)
    G = (rng.integers(-8, 8, (k, D)) / 4.0).astype(np.float32)
    W0 = (rng.integers(-8, 8, E * D) / 8.0).astype(np.float32)
    # k bags of one lookup each, all row 3
    rep = workloads.Batch(np.full(k, 3, np.int64), np.arange(k + 1, dtype=np.int64), None)
    W_rep, st_rep = W0.copy(), np.zeros(E, np.float32)
    _update(spec, W_rep, st_rep, rep, G)
    one_spec = workloads.custom([E], [D], "f32", B=1, optimizer=optimizer, lr=0.25, eps=0.0)
    one = workloads.Batch(np.array([3], np.int64), np.array([0, 1], np.int64), None)
    W_one, st_one = W0.copy(), np.zeros(E, np.float32)
    _update(one_spec, W_one, st_one, one, G.sum(axis=0, keepdims=True))
    assert np.array_equal(W_rep, W_one) and np.array_equal(st_rep, st_one)

    # versus k sequential per-lookup updates: equal for SGD (linear), different for Adagrad
    W_seq, st_seq = W0.copy(), np.zeros(E, np.float32)
    for j in range(k):
        _update(one_spec, W_seq, st_seq, one, G[j:j + 1])
    if optimizer == "sgd":
        assert np.array_equal(W_seq, W_rep)
    else:
        assert not np.array_equal(W_seq, W_rep)


def test_rowwise_adagrad_closed_form_two_steps():
    spec = workloads.custom([60, 25], [16, 8], "f32", B=24, lengths=("uniform_int", 1, 6),
                            optimizer="rowwise_adagrad", index_dist=("zipf", 1.1), lr=LR, eps=EPS)
    W0 = _np_weights(spec, seed=11)
    W = W0.copy()
    st = np.zeros(spec.sum_rows, np.float32)
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    woff = np.concatenate([[0], np.cumsum(np.array(spec.rows) * np.array(spec.dims))])
    m_expect = np.zeros(spec.sum_rows)
    for step in range(2):
        batch = workloads.batch(spec, seed=11, step=step)
        G = _np_grad(spec, seed=11, step=step)
        before = W.astype(np.float64).copy()
        _update(spec, W, st, batch, G)
        gam = _dense_AtG(spec, batch, G)
        for t in range(spec.T):
            D = spec.dims[t]
            gt = gam[woff[t]:woff[t + 1]].reshape(-1, D)
            dW = (W.astype(np.float64) - before)[woff[t]:woff[t + 1]].reshape(-1, D)
            hit = np.unique(batch.indices[batch.offsets[t * spec.B]:batch.offsets[(t + 1) * spec.B]])
            for r in hit:
                lin = roff[t] + r
                m_expect[lin] += np.mean(gt[r] ** 2)           # state accumulates the row mean of Gamma^2
                assert abs(st[lin] - m_expect[lin]) <= 2e-7 * m_expect[lin]
                rho = np.sqrt(m_expect[lin])
                # the step is parallel to -Gamma with length lr * |Gamma| / (rho + eps)
                want = -LR * gt[r] / (rho + EPS)
                # tolerance: one fp32 rounding of the stored weight
                scale = np.abs(before[woff[t] + r * D:woff[t] + (r + 1) * D]).max() + LR
                assert np.allclose(dW[r], want, rtol=0, atol=2.0 ** -23 * scale)
                if step == 0:
                    # from zero state: rms of the step equals lr * rho / (rho + eps)
                    assert abs(np.sqrt(np.mean(want ** 2)) - LR * rho / (rho + EPS)) <= 1e-12


def _torch_bag_loss(spec, batch, G, params, torch):
    """<G, forward(W)> through torch's own embedding_bag (sum pooling), one table at a time."""
    loss = 0.0
    for t in range(spec.T):
        lo, hi = int(batch.offsets[t * spec.B]), int(batch.offsets[(t + 1) * spec.B])
        off = torch.from_numpy(batch.offsets[t * spec.B:(t + 1) * spec.B + 1] - lo)
        idx = torch.from_numpy(batch.indices[lo:hi])
        p = None if batch.psw is None else torch.from_numpy(batch.psw[lo:hi].astype(np.float64))
        Y = torch.nn.functional.embedding_bag(idx, params[t], off, mode="sum", per_sample_weights=p,
                                              include_last_offset=True)
        loss = loss + (Y * torch.from_numpy(G[:, t:t + 1].astype(np.float64))).sum()
    return loss


@pytest.mark.parametrize("psw", [False, True], ids=["plain", "weighted"])
def test_rowwise_adagrad_at_dim_one_is_torch_adagrad(psw):
    # With one column per row, the row-wise Adagrad reading (state += mean over the row of
    # Gamma^2, then W -= lr * Gamma / (sqrt(state) + eps) with the updated state, state from
    # 0) is plain Adagrad, which torch.optim.Adagrad implements independently (lr_decay 0,
    # weight_decay 0, initial accumulator 0).  eps = 0.25 is large enough to tell
    # sqrt(m) + eps from sqrt(m + eps) by several percent, and the state is used after its
    # update (the other order divides the first step by eps alone).  Duplicate rows inside a
    # batch and rows left out of some steps are both present.  Each step starts torch from
    # the oracle's weights and state (both fp32-representable) and runs it in fp64; the
    # oracle rounds its fp64 result once to fp32, so the two agree to one fp32 rounding.
    import torch
    lr, eps = 0.05, 0.25
    spec = workloads.custom([40, 9], [1, 1], "f32", B=16, lengths=("uniform_int", 0, 6),
                            index_dist=("zipf", 1.4), psw=psw, optimizer="rowwise_adagrad",
                            key=280, lr=lr, eps=eps)
    roff = np.concatenate([[0], np.cumsum(spec.rows)])

    def params_from(W):
        return [torch.nn.Parameter(torch.from_numpy(W[roff[t]:roff[t + 1]].astype(np.float64))
                                   .reshape(-1, 1)) for t in range(spec.T)]

    def adagrad(params):
        return torch.optim.Adagrad(params, lr=lr, lr_decay=0, weight_decay=0,
                                   initial_accumulator_value=0, eps=eps)

    def flat(ts):
        return np.concatenate([t.detach().numpy().reshape(-1) for t in ts])

    W = _np_weights(spec, seed=21)
    st = np.zeros(spec.sum_rows, np.float32)
    chain = params_from(W)          # a torch-only trajectory over every step, never resynchronised
    chain_opt = adagrad(chain)
    skipped_rows_seen = False
    for step in range(4):
        batch = workloads.batch(spec, seed=21, step=step)
        G = _np_grad(spec, seed=21, step=step)
        params = params_from(W)
        opt = adagrad(params)
        for t, p in enumerate(params):
            opt.state[p]["sum"].copy_(torch.from_numpy(st[roff[t]:roff[t + 1]].astype(np.float64))
                                      .reshape(-1, 1))
        _torch_bag_loss(spec, batch, G, params, torch).backward()
        gamma = flat([p.grad for p in params])
        opt.step()
        _torch_bag_loss(spec, batch, G, chain, torch).backward()
        chain_opt.step()
        chain_opt.zero_grad()

        W_before, st_before = W.copy(), st.copy()
        _update(spec, W, st, batch, G)
        uniq, cnt = oracle.runs(spec.rows, spec.B, batch.indices, batch.offsets)
        assert (cnt > 1).any()                                   # duplicates in this batch
        untouched = np.setdiff1d(np.arange(spec.sum_rows), uniq)
        skipped_rows_seen |= bool((st_before[untouched] > 0).any())
        assert np.array_equal(W[untouched], W_before[untouched])
        assert np.array_equal(st[untouched], st_before[untouched])

        w_t, m_t = flat(params), flat([opt.state[p]["sum"] for p in params])
        assert np.all(np.abs(W - w_t) <= 2.0 ** -23 * np.abs(w_t)), f"weights, step {step}"
        assert np.all(np.abs(st - m_t) <= 2.0 ** -23 * m_t), f"state, step {step}"
        # fp32 rounding of the stored weights and state, carried over the steps
        assert np.all(np.abs(W - flat(chain)) <= 1e-6 * (np.abs(flat(chain)) + lr))
        # the readings rejected for the pages' silence land far outside that bound
        w0, g, m0, m1 = W_before[uniq].astype(np.float64), gamma[uniq], st_before[uniq], m_t[uniq]
        eps_inside = w0 - lr * g / np.sqrt(m1 + eps)
        state_after_use = w0 - lr * g / (np.sqrt(m0) + eps)
        for alt in (eps_inside, state_after_use):
            far = np.abs(alt - w_t[uniq]) > 1e3 * 2.0 ** -23 * np.abs(w_t[uniq])
            assert far.mean() > 0.5
    assert skipped_rows_seen                                     # some row with state sat out a step

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_low_precision_update_rounds_once_to_nearest(dtype):
    spec = workloads.custom([30], [8], dtype, B=10, lengths=("uniform_int", 1, 5), lr=LR)
    batch = workloads.batch(spec, seed=12)
    G = _np_grad(spec, seed=12)
    dt = workloads.oracle_dtype(dtype)
    W0 = _np_weights(spec, seed=12)
    W = W0.copy()
    _update(spec, W, None, batch, G)
    exact = oracle.widen(dt, W0) - LR * _dense_AtG(spec, batch, G)
    got = oracle.widen(dt, W)
    up = oracle.widen(dt, (W.astype(np.int64) + 1).astype(np.uint16))
    dn = oracle.widen(dt, np.where((W & 0x7FFF) == 0, W, W.astype(np.int64) - 1).astype(np.uint16))
    err = np.abs(got - exact)
    assert (err <= np.abs(up - exact)).all() and (err <= np.abs(dn - exact)).all()


def test_selected_rows_update_matches_full_update_on_those_rows():
    spec = workloads.custom([500, 80], [8, 4], "bf16", B=64, lengths=("uniform_int", 0, 12),
                            optimizer="rowwise_adagrad", index_dist=("zipf", 1.2), pooling="mean", psw=True)
    batch = workloads.batch(spec, seed=13)
    G = _np_grad(spec, seed=13)
    W0 = _np_weights(spec, seed=13)
    Wf, sf = W0.copy(), np.zeros(spec.sum_rows, np.float32)
    _update(spec, Wf, sf, batch, G)
    uniq, _ = oracle.runs(spec.rows, spec.B, batch.indices, batch.offsets)
    sel = np.sort(np.random.default_rng(0).choice(uniq, 40, replace=False))
    Ws, ss = W0.copy(), np.zeros(spec.sum_rows, np.float32)
    _update(spec, Ws, ss, batch, G, selected=sel)
    assert np.array_equal(ss[sel], sf[sel])
    changed = np.nonzero(ss)[0]
    assert np.array_equal(np.sort(changed), np.sort(sel[sf[sel] != 0]))
    # weights: selected rows equal the full update, other rows untouched
    roff = np.concatenate([[0], np.cumsum(spec.rows)])
    woff = np.concatenate([[0], np.cumsum(np.array(spec.rows) * np.array(spec.dims))])
    for lin in sel:
        t = int(np.searchsorted(roff, lin, side="right") - 1)
        D = spec.dims[t]
        a = woff[t] + (lin - roff[t]) * D
        assert np.array_equal(Ws[a:a + D], Wf[a:a + D])
    assert np.array_equal(np.nonzero(Ws != W0)[0], np.nonzero((Ws != W0) & (Wf != W0))[0])
