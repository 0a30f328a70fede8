"""Seeded random configurations against the CPU reference: table counts, row counts (from a
handful of rows, through tables small enough for the LDS forward, to 200k rows), widths,
storage dtypes, bag-length mixes (empty bags included), id skew, pooling, per-sample weights,
optimizer, id dtype, plain or grouped calls, and batches on both sides of 2^20 lookups (bucket-
local sort and counted LSD passes).  Each configuration runs two forward + backward_update steps
through the C ABI, checked as every parity test is (forward within tolerance, runs bit-exact,
updated rows within tolerance, untouched rows bit-identical, guard bands intact)."""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_parity import parity

pytestmark = pytest.mark.gpu

N_CONFIGS = 40


def _pick(rng, options):
    return options[int(rng.integers(0, len(options)))]


def _spec(i):
    rng = np.random.default_rng(9100 + i)
    big = i % 5 == 4                      # about 1.5 M lookups: counted passes
    dtype = _pick(rng, ["f32", "f16", "bf16"])
    T = int(rng.integers(1, 3 if big else 9))
    rows = [int(_pick(rng, [rng.integers(1, 20), rng.integers(20, 1025), rng.integers(1025, 200_000)]))
            for _ in range(T)]
    dims = ([int(_pick(rng, [4, 8, 12, 16, 32, 64, 100, 128, 256])) for _ in range(T)]
            if dtype == "f32" else [int(_pick(rng, [8, 16, 24, 32, 40, 64, 128])) for _ in range(T)])
    if big:
        B, lengths = 20000, ("uniform_int", 20, 60)
    else:
        B = int(rng.integers(1, 3000))
        lengths = _pick(rng, [("fixed", int(rng.integers(0, 20))),
                              ("uniform_int", 0, int(rng.integers(1, 60))),
                              ("poisson_clip", 10.0, 0, 40)])
    index_dist = _pick(rng, [("uniform",), ("zipf", 1.05), ("zipf", 1.3)])
    spec = workloads.custom(rows, dims, dtype, B=B, lengths=lengths, index_dist=index_dist,
                            pooling=_pick(rng, ["sum", "mean"]), psw=bool(rng.integers(0, 2)),
                            optimizer=_pick(rng, ["sgd", "rowwise_adagrad"]), key=9100 + i,
                            name=f"random{i}")
    idt = _pick(rng, [torch.int32, torch.int64])
    grouped = bool(rng.integers(0, 2))
    return spec, idt, grouped, big


@pytest.mark.timeout(600)
@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_config_parity(i):
    spec, idt, grouped, big = _spec(i)
    print(f"[random {i}] T={spec.T} rows={spec.rows} dims={spec.dims} {spec.dtype} B={spec.B} "
          f"{spec.lengths} {spec.index_dist} {spec.pooling} psw={spec.psw} {spec.optimizer} "
          f"{idt} grouped={grouped}", flush=True)
    parity(spec, seed=i, steps=2, index_dtype=idt, grouped=grouped,
           bag_sample=4000 if big else None, row_sample=5000 if big else None)
