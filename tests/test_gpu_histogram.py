"""GPU parity of the count-matrix (histogram, MFMA) forward for small 16-bit tables.

kimbodo.com/?p=28372, "What Happened": small tables that qualify are pooled through a
histogram and the matrix cores, next to the generic gather path.  The result is the pooled
gather itself (Y_t = diag(s) C_t W_t with C_t the bag-by-row count matrix), so the CPU
reference for it is the plain forward; the comparison rules are those of gpu_check.py.
"""
import numpy as np
import pytest
import torch

import oracle
import table_embedding_bag_amd as tbe
import workloads
from gpu_check import abs_bits, code, make_problem, pool
from test_gpu_parity import _hand_batch, parity

pytestmark = pytest.mark.gpu

FORCE, NO_HIST = tbe.FLAG_FORCE_HISTOGRAM, tbe.FLAG_NO_HISTOGRAM

HIST = [
    # several 64-column tiles (80 = 64 + 16, 256 = 4 x 64), rows not a multiple of 64,
    # a ragged last 256-bag tile, empty bags
    workloads.custom([64, 100, 1000, 1024], [16, 80, 64, 256], "bf16", B=300,
                     lengths=("uniform_int", 0, 12), key=301),
    # repeated rows inside bags and more than 2048 lookups per workgroup (several batches)
    workloads.custom([64, 700], [64, 32], "bf16", B=257, lengths=("uniform_int", 10, 30),
                     index_dist=("zipf", 1.2), pooling="mean", optimizer="rowwise_adagrad", key=302),
    workloads.custom([500, 33], [128, 16], "f16", B=70, lengths=("uniform_int", 0, 20),
                     pooling="mean", key=303),
    # bags on both sides of 256 lookups (bf16 counts are exact up to 256), hot rows
    workloads.custom([200], [64], "bf16", B=20, lengths=("uniform_int", 250, 262),
                     index_dist=("zipf", 1.3), key=304),
    # fp16 counts are exact up to 2048
    workloads.custom([100], [32], "f16", B=6, lengths=("uniform_int", 2040, 2056),
                     index_dist=("zipf", 1.5), pooling="mean", key=305),
    # bags longer than the ids a lane keeps in registers: the wave lists its lookups in
    # batches of 512 (up to 15 per wave here), 16 row chunks, a wave with only short bags
    workloads.custom([1024, 64, 300], [64, 32, 16], "bf16", B=300,
                     lengths=("uniform_int", 9, 120), index_dist=("zipf", 1.1), key=307),
]


@pytest.mark.parametrize("spec", HIST, ids=lambda s: f"{s.key}-{s.dtype}-{s.pooling}")
def test_forced_histogram_parity(spec):
    parity(spec, seed=3, steps=2, flags=FORCE)


def test_histogram_int32_indices():
    parity(HIST[0], seed=4, steps=1, index_dtype=torch.int32, flags=FORCE)


def test_routing_mixes_both_forwards():
    """With TBE_FLAG_HISTOGRAM, qualifying tables (bf16, <= 1024 rows, dims in 16-column
    tiles) take the count-matrix forward and the others the gather forward, in one call."""
    spec = workloads.custom([300, 5000, 64, 40], [32, 32, 24, 512], "bf16", B=130,
                            lengths=("uniform_int", 0, 10), key=306, optimizer="rowwise_adagrad")
    parity(spec, seed=5, steps=2, flags=tbe.FLAG_HISTOGRAM)


def test_histogram_routing_with_weights_uses_gather():
    """Per-sample weights rule the count-matrix forward out for the call (the counts would
    no longer be integers): the routed handle pools such a batch with the gather forward."""
    spec = workloads.custom([300, 64], [32, 64], "bf16", B=70, lengths=("uniform_int", 0, 10),
                            psw=True, pooling="mean", key=307)
    parity(spec, seed=8, steps=1, flags=tbe.FLAG_HISTOGRAM)


def test_histogram_and_gather_agree():
    spec = HIST[0]
    pa = make_problem(spec, seed=6, flags=FORCE)
    pb = make_problem(spec, seed=6, flags=NO_HIST)
    ya = pa.op.forward(spec.B, pa.idx, pa.off)
    yb = pb.op.forward(spec.B, pb.idx, pb.off)
    torch.cuda.synchronize()
    scale = oracle.forward(spec.rows, spec.dims, code(spec), pool(spec),
                           abs_bits(spec, workloads.storage_numpy(pa.W)), spec.B,
                           pa.batch.indices, pa.batch.offsets)
    assert np.all(np.abs(ya.cpu().numpy() - yb.cpu().numpy()) <= 2e-5 * scale + 1e-30)
    pa.op.close()
    pb.op.close()


def _dyadic_table(E, D):
    """Rows of multiples of 1/64 in [-1/8, 1/8): every sum of up to 2^12 of them is exact in
    fp32, so any summation order gives the same bits."""
    r = np.arange(E)[:, None]
    d = np.arange(D)[None, :]
    return (((r * 7 + d * 3) % 16) - 8).astype(np.float32) / 64.0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_count_limits_bit_exact(dtype):
    """Bags whose count of one row is exactly at the 16-bit limit (256 for bf16, 2048 for
    fp16), one past it (pooled by the fallback gather), and ordinary bags; dyadic weights
    make the sums exact, so the output must equal the reference bit for bit."""
    cap = 256 if dtype == "bf16" else 2048
    E, D = 130, 48
    Wn = _dyadic_table(E, D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    W = torch.from_numpy(Wn.reshape(-1)).to(tdt).cuda()
    bags = [[[5] * cap, [5] * cap + [7], [3, 3, 129], [], [0] * (cap - 1) + [1] * 3, [64, 63, 65]]]
    batch = _hand_batch(1, len(bags[0]), bags)
    op = tbe.TBE([E], [D], W, flags=FORCE)
    idx = torch.from_numpy(batch.indices).cuda()
    off = torch.from_numpy(batch.offsets).cuda()
    Y = op.forward(len(bags[0]), idx, off).cpu().numpy()
    for b, bag in enumerate(bags[0]):
        want = Wn[bag].astype(np.float64).sum(axis=0) if bag else np.zeros(D)
        assert np.array_equal(Y[b], want.astype(np.float32)), f"bag {b}"
    op.close()


def test_forced_histogram_rejects_per_sample_weights():
    spec = HIST[0]
    pb = make_problem(spec, seed=7, flags=FORCE)
    psw = torch.rand(pb.batch.N, device="cuda")
    with pytest.raises(tbe.TBEError, match="UNSUPPORTED"):
        pb.op.forward(spec.B, pb.idx, pb.off, psw)
    pb.op.close()


@pytest.mark.timeout(900)
def test_count_matrix_forward_on_the_64_small_tables_at_full_size():
    """Every table of the many-small-tables batch (64 bf16 tables of 64..1024 rows, dim 64,
    B = 32768 bags of 8 uniform lookups: 16.8 M lookups) through the count-matrix forward,
    two steps with the backward in between; sampled bags and rows."""
    parity(workloads.config(5), seed=0, steps=2, bag_sample=20000, row_sample=50000, flags=FORCE)
