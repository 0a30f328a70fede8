"""Shared parity machinery for the GPU tests: run the HIP library through its
C ABI on seeded inputs and compare every result with the CPU reference.

Comparison rules (tolerances relative to the absolute-sum scale, since sums of
signed values may cancel):
  forward       |Y - Y_ref| <= rtol * s_k * sum_i |p_i W[x_i, d]|
                rtol = 1e-5 for fp32 storage, 1e-2 for fp16 / bf16 storage;
                every storage dtype is also held to 1e-5, as both sides read the
                same stored values and accumulate in fp32 or better.
  runs          unique row ids, run lengths and their count: bit-exact.
  fp32 weights  |W - W_ref| <= 1e-5 * (|W_old| + max_d |W_ref - W_old| over the row)
  fp16 / bf16   within one unit in the last place of the storage dtype at W_ref (plus
                the fp32 term above where the new value nearly cancels), and at least
                99.9% of the compared elements bit-equal to the reference's rounding.
  state         |m - m_ref| <= 1e-5 * m_ref.
  other rows    bit-identical weights and state.
  guard bands   the weights, the optimizer state and the outputs sit inside larger
                buffers whose GUARD elements before and after hold a known pattern,
                which must be intact after every call (a write past either end fails).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import oracle
import table_embedding_bag_amd as tbe
import workloads

DEV = "cuda"

GUARD = 4096          # elements of known pattern on each side of a guarded buffer
_PATTERN = {1: 0x5A, 2: 0x5A5A, 4: 0x5A5A5A5A}
_INT_VIEW = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


def guarded_empty(shape, dtype, device=DEV):
    """(buffer, view): an uninitialised tensor of `shape` inside a buffer whose GUARD
    elements before and after hold a fixed bit pattern (checked by guards_intact)."""
    numel = int(np.prod(shape)) if len(shape) else 1
    buf = torch.empty(numel + 2 * GUARD, dtype=dtype, device=device)
    size = buf.element_size()
    bits = buf.view(_INT_VIEW[size])
    pat = _PATTERN[size] if size != 2 else np.int16(np.uint16(_PATTERN[2]).view(np.int16))
    bits[:GUARD].fill_(int(pat))
    bits[GUARD + numel:].fill_(int(pat))
    return buf, buf[GUARD:GUARD + numel].view(shape)


def guarded_copy(t):
    buf, view = guarded_empty(tuple(t.shape), t.dtype, t.device)
    view.copy_(t)
    return buf, view


def guards_intact(buf) -> bool:
    size = buf.element_size()
    bits = buf.view(_INT_VIEW[size])
    pat = _PATTERN[size] if size != 2 else np.int16(np.uint16(_PATTERN[2]).view(np.int16))
    head, tail = bits[:GUARD], bits[bits.numel() - GUARD:]
    return bool((head == int(pat)).all().item()) and bool((tail == int(pat)).all().item())


def code(spec):
    return workloads.oracle_dtype(spec.dtype)


def pool(spec):
    return oracle.POOL_MEAN if spec.pooling == "mean" else oracle.POOL_SUM


def opt(spec):
    return oracle.OPT_ROWWISE_ADAGRAD if spec.optimizer == "rowwise_adagrad" else oracle.OPT_SGD


def abs_bits(spec, W: np.ndarray) -> np.ndarray:
    """|W| of raw storage bits (sign bit cleared)."""
    if spec.dtype == "f32":
        return np.abs(W)
    return W & np.uint16(0x7FFF)


def layout(spec):
    rows = np.array(spec.rows, np.int64)
    dims = np.array(spec.dims, np.int64)
    return (np.concatenate([[0], np.cumsum(rows * dims)]), np.concatenate([[0], np.cumsum(rows)]),
            np.concatenate([[0], np.cumsum(dims)]))


@dataclasses.dataclass
class Problem:
    spec: workloads.Spec
    batch: workloads.Batch
    W: torch.Tensor                 # device weights (updated in place by the library)
    state: Optional[torch.Tensor]
    op: tbe.TBE
    idx: torch.Tensor
    off: torch.Tensor
    psw: Optional[torch.Tensor]
    guards: list = dataclasses.field(default_factory=list)   # buffers with guard bands

    def check_guards(self, *extra):
        for buf in list(self.guards) + list(extra):
            assert guards_intact(buf), "a write landed outside its buffer (guard band changed)"


def make_problem(spec, seed=0, step=0, index_dtype=torch.int64, batch=None, flags=0) -> Problem:
    batch = batch if batch is not None else workloads.batch(spec, seed=seed, step=step)
    wbuf, W = guarded_copy(workloads.weights(spec, seed=seed, device=DEV))
    guards = [wbuf]
    state = None
    if spec.optimizer == "rowwise_adagrad":
        sbuf, state = guarded_empty((spec.sum_rows,), torch.float32)
        state.zero_()
        guards.append(sbuf)
    op = tbe.TBE(spec.rows, spec.dims, W, state, pooling=spec.pooling, optimizer=spec.optimizer,
                 flags=flags)
    return Problem(spec, batch, W, state, op, *to_device(batch, index_dtype), guards=guards)


def to_device(batch, index_dtype=torch.int64):
    idx = torch.from_numpy(batch.indices).to(DEV, index_dtype)
    off = torch.from_numpy(batch.offsets).to(DEV, index_dtype)
    psw = torch.from_numpy(batch.psw).to(DEV) if batch.psw is not None else None
    return idx, off, psw


def check_forward(pb: Problem, Y: torch.Tensor, W_host: np.ndarray, bag_sample=None, dev=None):
    """Compare the GPU output with the reference on all bags (or a sample of bag ids).
    dev: per linear row, the deviation the GPU's weights may carry from earlier steps."""
    spec, batch = pb.spec, pb.batch
    Yh = Y.cpu().numpy()
    _, _, doff = layout(spec)
    if bag_sample is None:
        ref = oracle.forward(spec.rows, spec.dims, code(spec), pool(spec), W_host, spec.B,
                             batch.indices, batch.offsets, batch.psw)
        scale = oracle.forward(spec.rows, spec.dims, code(spec), pool(spec), abs_bits(spec, W_host),
                               spec.B, batch.indices, batch.offsets,
                               None if batch.psw is None else np.abs(batch.psw))
        got = Yh
        ids = np.arange(spec.T * spec.B)
    else:
        ids = np.asarray(bag_sample, np.int64)
        ref = np.concatenate(oracle.forward_bags(spec.rows, spec.dims, code(spec), pool(spec), W_host,
                                                 spec.B, batch.indices, batch.offsets, batch.psw, ids))
        scale = np.concatenate(oracle.forward_bags(
            spec.rows, spec.dims, code(spec), pool(spec), abs_bits(spec, W_host), spec.B,
            batch.indices, batch.offsets, None if batch.psw is None else np.abs(batch.psw), ids))
        got = np.concatenate([Yh[k % spec.B, doff[k // spec.B]:doff[k // spec.B + 1]] for k in ids])
    carried = 0.0
    if dev is not None and dev.any():
        per_bag = forward_deviation(spec, pb.batch, dev)
        if bag_sample is None:
            carried = np.concatenate([np.repeat(per_bag[t * spec.B:(t + 1) * spec.B, None],
                                                spec.dims[t], axis=1) for t in range(spec.T)], axis=1)
        else:
            carried = np.concatenate([np.full(spec.dims[k // spec.B], per_bag[k]) for k in ids])
    err = np.abs(got - ref)
    rel = err / (scale + 1e-30)
    rtol = 1e-5 if spec.dtype == "f32" else 1e-2
    assert np.isfinite(got).all()
    assert (err <= rtol * scale + carried + 1e-30).all(), f"forward: max rel err {rel.max():.3e} > {rtol}"
    assert (err <= 1e-5 * scale + carried + 1e-30).all(), f"forward: max rel err {rel.max():.3e} > 1e-5"
    return float(rel.max())


def gpu_runs(pb: Problem, n):
    u = torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    c = torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    k = torch.zeros(1, dtype=torch.int32, device=DEV)
    return u, c, k


def check_runs(pb: Problem, runs):
    spec, batch = pb.spec, pb.batch
    uniq, cnt = oracle.runs(spec.rows, spec.B, batch.indices, batch.offsets)
    U = int(runs[2].item())
    assert U == uniq.size, f"U {U} != {uniq.size}"
    assert np.array_equal(runs[0][:U].cpu().numpy().astype(np.int64), uniq)
    assert np.array_equal(runs[1][:U].cpu().numpy().astype(np.int64), cnt)
    return uniq, cnt


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in units of the storage format between 16-bit codes (monotone ordering)."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def rows_of(spec, flat, linear_ids):
    """{table: [n_t, D_t] raw storage rows} of the given linear row ids, from a
    flat host array or a flat device tensor (gathered on the device)."""
    woff, roff, _ = layout(spec)
    ids = np.asarray(linear_ids, np.int64)
    tab = np.searchsorted(roff, ids, side="right") - 1
    out = {}
    for t in np.unique(tab):
        D = spec.dims[t]
        r = ids[tab == t] - roff[t]
        el = woff[t] + r[:, None] * D + np.arange(D)[None, :]
        if isinstance(flat, torch.Tensor):
            out[int(t)] = workloads.storage_numpy(flat[torch.from_numpy(el.reshape(-1)).to(flat.device)]).reshape(-1, D)
        else:
            out[int(t)] = flat[el]
    return out


def spacing(spec, bits: np.ndarray) -> np.ndarray:
    """Gap between the stored value and the next code away from zero (fp16 / bf16)."""
    dt = code(spec)
    mag = (bits & np.uint16(0x7FFF)).astype(np.int64)
    lo = np.minimum(mag, 0x7BFE if spec.dtype == "f16" else 0x7F7E)
    return oracle.widen(dt, (lo + 1).astype(np.uint16)) - oracle.widen(dt, lo.astype(np.uint16))


def values(spec, rows: np.ndarray) -> np.ndarray:
    """Stored rows as float64 values."""
    if spec.dtype == "f32":
        return rows.astype(np.float64)
    return oracle.widen(code(spec), rows.reshape(-1)).reshape(rows.shape)


def update_allowance(spec, before: dict, after: dict) -> dict:
    """Per element: how far the GPU's new weights may be from the reference's after
    one update of these rows from identical inputs.

    The update is computed in fp32 on the GPU and in fp64 by the reference, so
    both differ by fp32-level rounding of W_old - step * Gamma, bounded by
    1e-5 * (|W_old| + max over the row of |W_new - W_old|); fp16 / bf16 storage
    adds one rounding to the storage grid (one unit in the last place at the
    reference value).  Where the new value nearly cancels, the storage grid is
    much finer than the fp32-level term, so a 'one ulp' bound alone is wrong."""
    out = {}
    for t, f in after.items():
        o, fv = values(spec, before[t]), values(spec, f)
        a = 1e-5 * (np.abs(o) + np.abs(fv - o).max(axis=1, keepdims=True))
        if spec.dtype != "f32":
            a = a + spacing(spec, f).reshape(f.shape)
        out[t] = a
    return out


def check_update(spec, ids, before: dict, ref: dict, gpu: dict, dev_old: np.ndarray,
                 st_ref=None, st_gpu=None, counts=None):
    """|W_gpu - W_ref| <= (allowed deviation carried in from earlier steps) + (one update's
    allowance); state within 1e-5 relative.  ids: sorted linear ids of the compared rows."""
    _, roff, _ = layout(spec)
    worst = 0.0
    allow = update_allowance(spec, before, ref)
    tab = np.searchsorted(roff, ids, side="right") - 1
    equal = compared = 0
    for t, f in ref.items():
        lin = ids[tab == t]
        g = gpu[t]
        fv, gv = values(spec, f), values(spec, g)
        err = np.abs(gv - fv)
        lim = dev_old[lin][:, None] + allow[t]
        ratio = err / (lim + 1e-38)
        if not (err <= lim).all():
            worst_rows = np.argsort(ratio.max(axis=1))[-5:]
            msg = [f"table {t}: weight error up to {ratio.max():.3f} x allowed"]
            for i in worst_rows:
                d = int(np.argmax(ratio[i]))
                c = "" if counts is None else f" hits={counts.get(int(lin[i]), '?')}"
                msg.append(f"  row {lin[i]}{c} col {d}: gpu {gv[i, d]:.6e} ref {fv[i, d]:.6e} "
                           f"err {err[i, d]:.3e} allowed {lim[i, d]:.3e}")
            raise AssertionError("\n".join(msg))
        worst = max(worst, float(ratio.max()))
        equal += int((g == f).sum())
        compared += g.size
    if spec.dtype != "f32" and compared:
        # both sides round once to the storage grid; they differ only where the fp32
        # rounding of the GPU's update crosses a rounding boundary of the 16-bit grid
        assert compared - equal <= 0.001 * compared + 1, \
            f"only {equal}/{compared} 16-bit weights bit-equal to the reference's rounding"
    if st_ref is not None:
        m, mr = st_gpu[ids], st_ref[ids]
        assert (np.abs(m - mr) <= 1e-5 * mr + 1e-30).all(), "state mismatch"
    return worst


def carry_deviation(spec, dev: np.ndarray, ids, before: dict, after: dict) -> None:
    """dev[row] += largest allowance of one update over the row (in place)."""
    _, roff, _ = layout(spec)
    tab = np.searchsorted(roff, ids, side="right") - 1
    for t, a in update_allowance(spec, before, after).items():
        lin = ids[tab == t]
        dev[lin] += a.max(axis=1)


def forward_deviation(spec, batch, dev: np.ndarray) -> np.ndarray:
    """Per bag: s_k * sum_i |p_i| dev[row_i], the effect of allowed weight deviations."""
    _, roff, _ = layout(spec)
    nb = spec.T * spec.B
    lens = np.diff(batch.offsets)
    bag = np.repeat(np.arange(nb), lens)
    lin = roff[bag // spec.B] + batch.indices
    v = dev[lin] * (1.0 if batch.psw is None else np.abs(batch.psw.astype(np.float64)))
    out = np.zeros(nb)
    np.add.at(out, bag, v)
    if spec.pooling == "mean":
        out = np.where(lens > 0, out / np.maximum(lens, 1), 0.0)
    return out


def run_step(pb: Problem, G: torch.Tensor, lr=None, eps=None, with_runs=True, grouped=False):
    """backward_update of the problem's batch (grouped: the variant that reuses the grouping a
    forward_group call left in the handle's workspace)."""
    spec = pb.spec
    runs = gpu_runs(pb, pb.batch.N) if with_runs else None
    update = pb.op.backward_update_grouped if grouped else pb.op.backward_update
    update(spec.B, pb.idx, pb.off, pb.psw, G, spec.lr if lr is None else lr,
           spec.eps if eps is None else eps, runs)
    torch.cuda.synchronize()
    return runs


def reference_update(pb: Problem, W_host: np.ndarray, st_host, G_host, selected=None):
    spec, batch = pb.spec, pb.batch
    oracle.backward_update(spec.rows, spec.dims, code(spec), pool(spec), opt(spec), W_host, st_host,
                           spec.B, batch.indices, batch.offsets, batch.psw, G_host,
                           float(np.float32(spec.lr)), float(np.float32(spec.eps)), selected)


def untouched_identical(spec, before: dict, gpu: dict, st_before=None, st_gpu=None, ids=None):
    """Rows no lookup hit keep bit-identical weights (and state)."""
    for t in before:
        assert np.array_equal(before[t], gpu[t]), f"table {t}: an untouched row changed"
    if st_before is not None:
        assert np.array_equal(st_before[ids], st_gpu[ids]), "untouched state changed"
