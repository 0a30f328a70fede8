"""GPU parity of the count-matrix backward for small tables (TBE_FLAG_COUNT_BACKWARD):
the summed row gradients Gamma_t = C_t^T G_t of every table on the matrix cores (G split
exactly into three bf16 parts, fp32 sums in a fixed order), then one optimizer update per
touched row, with no sort.  It extends to the backward the histogram and tensor-core path
that kimbodo.com/?p=28372, "What Happened", gives small tables in the forward.  The CPU
reference is the plain one-update-per-row backward; comparison rules as in gpu_check.py
(runs bit-exact, weights within the update tolerance, at least 99.9% of 16-bit weights
bit-equal, untouched rows bit-identical, guard bands intact)."""
import numpy as np
import pytest
import torch

import table_embedding_bag_amd as tbe
import workloads
from gpu_check import make_problem, to_device
from test_gpu_parity import _hand_batch, parity

pytestmark = pytest.mark.gpu

CB = tbe.FLAG_COUNT_BACKWARD

SMALL = [
    # several 64-column slices (80 = 64 + 16, 256 = 4 x 64), rows not a multiple of 64
    # or of 256, empty bags, B not a multiple of 32
    workloads.custom([64, 100, 1000, 1024], [16, 80, 64, 256], "f32", B=300,
                     lengths=("uniform_int", 0, 12), key=701),
    workloads.custom([700, 64], [64, 32], "bf16", B=257, lengths=("uniform_int", 1, 30),
                     index_dist=("zipf", 1.2), pooling="mean", optimizer="rowwise_adagrad",
                     key=702),
    workloads.custom([1024, 33], [128, 16], "f16", B=70, lengths=("uniform_int", 0, 20),
                     optimizer="rowwise_adagrad", key=703),
    # few bags: most bag slices empty
    workloads.custom([500], [32], "f32", B=5, lengths=("uniform_int", 0, 9), key=704),
    # bags longer than 256 lookups with hot rows: counts above 256 in one bag
    workloads.custom([200], [64], "bf16", B=20, lengths=("uniform_int", 250, 700),
                     index_dist=("zipf", 1.3), key=705),
    # degenerate and edge row counts: a one-row table (every lookup on row 0), one row
    # short of and one past a wave's 64 rows, one row short of the 1024-row limit
    workloads.custom([1, 63, 65, 1023], [16, 32, 48, 64], "f32", B=97,
                     lengths=("uniform_int", 0, 16), optimizer="rowwise_adagrad", key=708),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: f"{s.key}-{s.dtype}-{s.pooling}-{s.optimizer}")
def test_count_backward_parity(spec):
    parity(spec, seed=1, steps=2, flags=CB)


def test_count_backward_grouped_and_int32():
    parity(SMALL[1], seed=2, steps=2, flags=CB, grouped=True)
    parity(SMALL[0], seed=3, steps=1, flags=CB, index_dtype=torch.int32)


def test_one_row_hit_a_thousand_times_in_one_bag():
    # a count of 1000 in a single bag is counted in passes of 256 positions
    E, B = 40, 64
    rng = np.random.default_rng(4)
    bags = [[list(rng.integers(0, E, rng.integers(0, 9))) for _ in range(B)]]
    bags[0][3] = [7] * 1000 + [8] * 300
    batch = _hand_batch(1, B, bags)
    for opt in ("sgd", "rowwise_adagrad"):
        spec = workloads.custom([E], [48], "f32", B=B, optimizer=opt, key=706)
        parity(spec, seed=5, steps=1, batches=[batch], flags=CB)


def test_weighted_calls_take_the_sort_path():
    spec = workloads.custom([300, 64], [32, 64], "bf16", B=100, lengths=("uniform_int", 0, 10),
                            psw=True, pooling="mean", optimizer="rowwise_adagrad", key=707)
    parity(spec, seed=6, steps=2, flags=CB)


def test_count_backward_is_deterministic():
    spec = SMALL[1]
    batch = workloads.batch(spec, seed=7)
    outs = []
    for _ in range(2):
        pb = make_problem(spec, seed=7, batch=batch, flags=CB)
        G = workloads.grad_output(spec, seed=7, device="cuda")
        pb.op.backward_update(spec.B, pb.idx, pb.off, None, G, spec.lr, spec.eps)
        torch.cuda.synchronize()
        outs.append((pb.W.clone(), pb.state.clone()))
        pb.op.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.timeout(900)
def test_count_backward_on_the_64_small_tables_at_full_size():
    """The many-small-tables batch (64 bf16 tables of 64..1024 rows, dim 64, B = 32768 bags
    of 8 uniform lookups: 16.8 M lookups, 97% of them in rows hit at least 256 times), two
    steps, sampled bags and rows."""
    parity(workloads.config(5), seed=0, steps=2, bag_sample=20000, row_sample=50000, flags=CB)
