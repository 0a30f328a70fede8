"""Seeded synthetic inputs for table-batched-embedding workloads.

This module only draws random numbers: table sizes, bag lengths, row ids,
per-sample weights, table values and upstream gradients.  It holds none of
the arithmetic of the method itself (no pooling, no grouping, no update), so
the GPU library and the CPU reference can both consume its output.

Recipe (where the sources leave a choice open, the plainest reading is taken):

* Host draws use numpy PCG64 with ``SeedSequence(seed, spawn_key=(workload,
  table, purpose, step))``, so every (table, purpose, step) has its own stream
  and the arrays do not depend on the order in which they are requested.
* Row ids are table-local.  "uniform" draws uniformly in ``[0, E_t)``;
  ``("zipf", a)`` draws a rank ``k`` in ``1..E_t`` with probability
  proportional to ``k**-a`` (inverse CDF of the finite distribution) and maps
  it through a seeded random permutation of the table's rows, so the hot rows
  are scattered over the table.
* Offsets are CSR with a trailing total, bags table-major (bag ``t*B + b``).
* Table values are ``N(0, 0.01**2)`` drawn in fp32 with a seeded torch
  generator on the device that will hold them, then rounded to the storage
  dtype (torch's conversion rounds to nearest even).  Upstream gradients are
  ``N(0, 1)`` fp32, drawn the same way, fresh for every step.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional, Tuple

import numpy as np

# purposes of the random streams
_LEN, _IDX, _PERM, _PSW, _ROWS, _WEIGHTS, _GRAD = 1, 2, 3, 4, 5, 6, 7

DTYPES = ("f32", "f16", "bf16")
POOLINGS = ("sum", "mean")
OPTIMIZERS = ("sgd", "rowwise_adagrad")


@dataclasses.dataclass(frozen=True)
class Spec:
    """A workload: table shapes plus how batches are drawn."""

    name: str
    key: int                      # workload id used in the seed streams
    rows: Tuple[int, ...]         # E_t
    dims: Tuple[int, ...]         # D_t
    dtype: str                    # storage dtype of all tables
    B: int                        # bags per table
    lengths: tuple                # ("fixed", L) | ("uniform_int", lo, hi) | ("poisson_clip", lam, lo, hi)
    index_dist: tuple             # ("uniform",) | ("zipf", alpha)
    pooling: str = "sum"
    psw: bool = False
    optimizer: str = "sgd"
    lr: float = 0.01
    eps: float = 1e-8
    weight_std: float = 0.01

    @property
    def T(self) -> int:
        return len(self.rows)

    @property
    def sum_dims(self) -> int:
        return int(sum(self.dims))

    @property
    def sum_rows(self) -> int:
        return int(sum(self.rows))

    @property
    def num_weights(self) -> int:
        return int(sum(int(e) * int(d) for e, d in zip(self.rows, self.dims)))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _torch_seed(seed: int, *key: int) -> int:
    return int(np.random.SeedSequence(seed, spawn_key=tuple(key)).generate_state(1, np.uint64)[0]
               & 0x7FFF_FFFF_FFFF_FFFF)


def config(n: int, seed: int = 0) -> Spec:
    """The five benchmark workloads (1-based), with all random shapes drawn."""
    if n == 1:
        return Spec("tiny: T=2 E=1000 D=16 fp32 B=64 L=4 uniform sum SGD", 1,
                    (1000, 1000), (16, 16), "f32", 64, ("fixed", 4), ("uniform",),
                    optimizer="sgd")
    if n == 2:
        return Spec("T=8 E=100000 D=128 fp32 B=2048 L~U{1..32} Zipf(1.05) sum rowwise-Adagrad", 2,
                    (100_000,) * 8, (128,) * 8, "f32", 2048, ("uniform_int", 1, 32),
                    ("zipf", 1.05), optimizer="rowwise_adagrad")
    if n == 3:
        rng = _rng(seed, 3, 0, _ROWS)
        rows = tuple(int(x) for x in np.floor(np.exp(rng.uniform(np.log(1e4), np.log(1e7), 32))))
        dims = tuple((32, 64, 128, 256)[t % 4] for t in range(32))
        return Spec("mixed: T=32 E~logU[1e4,1e7] D cycling 32..256 bf16 B=8192 "
                    "L~clip(Poisson(20),0,100) Zipf(1.1) mean psw rowwise-Adagrad", 3,
                    rows, dims, "bf16", 8192, ("poisson_clip", 20.0, 0, 100), ("zipf", 1.1),
                    pooling="mean", psw=True, optimizer="rowwise_adagrad")
    if n == 4:
        return Spec("hot rows: T=4 E=1e6 D=128 fp16 B=16384 L=64 Zipf(1.3) sum rowwise-Adagrad", 4,
                    (1_000_000,) * 4, (128,) * 4, "f16", 16384, ("fixed", 64), ("zipf", 1.3),
                    optimizer="rowwise_adagrad")
    if n == 5:
        rng = _rng(seed, 5, 0, _ROWS)
        rows = tuple(int(x) for x in rng.integers(64, 1024, size=64, endpoint=True))
        return Spec("small tables: T=64 E~U{64..1024} D=64 bf16 B=32768 L=8 uniform sum SGD", 5,
                    rows, (64,) * 64, "bf16", 32768, ("fixed", 8), ("uniform",), optimizer="sgd")
    raise ValueError(f"no workload {n}")


def custom(rows, dims, dtype="f32", B=8, lengths=("uniform_int", 0, 6), index_dist=("uniform",),
           pooling="sum", psw=False, optimizer="sgd", key=100, name="custom", lr=0.01,
           eps=1e-8) -> Spec:
    return Spec(name, key, tuple(int(r) for r in rows), tuple(int(d) for d in dims), dtype, int(B),
                tuple(lengths), tuple(index_dist), pooling, psw, optimizer, lr, eps)


def _lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "fixed":
        return np.full(spec.B, int(spec.lengths[1]), dtype=np.int64)
    if kind == "uniform_int":
        return rng.integers(spec.lengths[1], spec.lengths[2], size=spec.B, endpoint=True).astype(np.int64)
    if kind == "poisson_clip":
        lam, lo, hi = spec.lengths[1:]
        return np.clip(rng.poisson(lam, size=spec.B), lo, hi).astype(np.int64)
    raise ValueError(kind)


@functools.lru_cache(maxsize=256)
def _zipf_cdf(E: int, alpha: float) -> np.ndarray:
    w = np.arange(1, E + 1, dtype=np.float64) ** (-alpha)
    c = np.cumsum(w)
    return c / c[-1]


@functools.lru_cache(maxsize=256)
def _permutation(seed: int, key: int, t: int, E: int) -> np.ndarray:
    return _rng(seed, key, t, _PERM).permutation(E).astype(np.int64)


def _rows_for(spec: Spec, seed: int, t: int, n: int, rng: np.random.Generator) -> np.ndarray:
    E = spec.rows[t]
    if spec.index_dist[0] == "uniform":
        return rng.integers(0, E, size=n, dtype=np.int64)
    if spec.index_dist[0] == "zipf":
        cdf = _zipf_cdf(E, float(spec.index_dist[1]))
        rank = np.searchsorted(cdf, rng.random(n), side="right")
        np.minimum(rank, E - 1, out=rank)
        return _permutation(seed, spec.key, t, E)[rank]
    raise ValueError(spec.index_dist)


@dataclasses.dataclass
class Batch:
    indices: np.ndarray           # int64 [N], table-local row ids
    offsets: np.ndarray           # int64 [T*B+1]
    psw: Optional[np.ndarray]     # float32 [N] or None

    @property
    def N(self) -> int:
        return int(self.indices.size)


def batch(spec: Spec, seed: int = 0, step: int = 0) -> Batch:
    """One seeded batch: bag lengths, row ids and (if the workload has them) per-sample weights."""
    lens, idx, psw = [], [], []
    for t in range(spec.T):
        L = _lengths(spec, _rng(seed, spec.key, t, _LEN, step))
        n = int(L.sum())
        lens.append(L)
        idx.append(_rows_for(spec, seed, t, n, _rng(seed, spec.key, t, _IDX, step)))
        if spec.psw:
            psw.append(_rng(seed, spec.key, t, _PSW, step).random(n, dtype=np.float32))
    lengths = np.concatenate(lens)
    offsets = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    indices = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    return Batch(indices, offsets, np.concatenate(psw) if spec.psw else None)


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def weights(spec: Spec, seed: int = 0, device="cpu"):
    """Flat table storage (1-D torch tensor of the storage dtype) on ``device``."""
    import torch
    out = torch.empty(spec.num_weights, dtype=torch_dtype(spec.dtype), device=device)
    pos = 0
    for t in range(spec.T):
        n = spec.rows[t] * spec.dims[t]
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, spec.key, t, _WEIGHTS))
        chunk = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        chunk.mul_(spec.weight_std)
        out[pos:pos + n].copy_(chunk)
        pos += n
        del chunk
    return out


def grad_output(spec: Spec, seed: int = 0, step: int = 0, device="cpu"):
    """Upstream gradient [B, sum dims] fp32 on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, spec.key, 0, _GRAD, step))
    return torch.randn((spec.B, spec.sum_dims), generator=g, device=device, dtype=torch.float32)


def storage_numpy(t) -> np.ndarray:
    """Raw bits of a torch storage tensor as numpy (float32, or uint16 for fp16/bf16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def oracle_dtype(dtype: str) -> int:
    return {"f32": 0, "f16": 1, "bf16": 2}[dtype]
