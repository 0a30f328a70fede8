"""Pins of the oracle's storage conversions (fp16 / bf16 <-> float).

Tables may be stored in fp16 or bf16 ("Optimizing Recommendation Systems with
FBTriton Table Batched Embeddings", "Pro Tips for TBE Scaling") and are
accumulated at a higher precision (kimbodo.com/?p=28372, "What Happened").
The oracle's conversions are written from the IEEE-754 definitions; here they
are checked exhaustively against torch's CPU conversions and, for inputs with
more precision than fp32, against a brute-force nearest-value search.
"""
import numpy as np
import pytest
import torch

import oracle

DT = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_widen_all_bit_patterns(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(dtype, bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(DT[dtype]).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_widen_f32_is_identity():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen(oracle.F32, x), x.astype(np.float64))


def _fp32_probe_values():
    rng = np.random.default_rng(7)
    # random bit patterns over every exponent, both signs
    raw = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    vals = raw.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # exact ties for bf16 (low 16 bits = 0x8000) and for fp16 around 1.0 and in the subnormal range
    ties_bf16 = ((rng.integers(0, 1 << 16, size=5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    k = rng.integers(-2048, 2048, size=5000)
    ties_f16 = ((2 * k + 1) * 2.0 ** -11).astype(np.float32)          # halfway between fp16 values near 1
    ties_f16_sub = ((2 * k + 1) * 2.0 ** -25).astype(np.float32)      # halfway between fp16 subnormals
    edges = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, -65520.0, 6.0e-8, 2.0 ** -24,
                      2.0 ** -25, 2.0 ** -26, 3.0e38, 3.4e38, 1.0e-40, -1.0e-45,
                      np.finfo(np.float32).max, np.finfo(np.float32).tiny], dtype=np.float32)
    return np.concatenate([vals, ties_bf16[np.isfinite(ties_bf16)], ties_f16, ties_f16_sub, edges])


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_narrow_matches_torch_on_fp32_inputs(dtype):
    # fp32 -> double is exact, so torch's fp32 -> fp16/bf16 conversion is the reference
    x = _fp32_probe_values()
    ours = oracle.narrow(dtype, x.astype(np.float64))
    ref = torch.from_numpy(x).to(DT[dtype]).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_narrow_nan_and_inf(dtype):
    out = oracle.narrow(dtype, np.array([np.nan, np.inf, -np.inf]))
    back = oracle.widen(dtype, out)
    assert np.isnan(back[0]) and back[1] == np.inf and back[2] == -np.inf


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_narrow_is_nearest_even_for_double_inputs(dtype):
    # inputs with more than fp32 precision: brute-force check against both neighbours
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20_000) * np.exp2(rng.integers(-20, 12, size=20_000))
    bits = oracle.narrow(dtype, x).astype(np.int64)
    got = oracle.widen(dtype, bits.astype(np.uint16))
    finite = np.isfinite(got)
    # neighbours: the adjacent codes (same sign, magnitude +-1 ulp)
    up = oracle.widen(dtype, (bits + 1).astype(np.uint16))
    dn = oracle.widen(dtype, np.where((bits & 0x7FFF) == 0, bits, bits - 1).astype(np.uint16))
    err = np.abs(got - x)
    for nb in (up, dn):
        ok = ~np.isfinite(nb) | (err <= np.abs(nb - x))
        assert ok[finite].all()
    # ties go to the even code
    tie = finite & np.isfinite(up) & (err == np.abs(up - x))
    assert ((bits[tie] & 1) == 0).all()


def test_narrow_f32_matches_numpy():
    x = np.random.default_rng(5).standard_normal(10_000) * 1e3
    ours = oracle.narrow(oracle.F32, x).view(np.float32)
    assert np.array_equal(ours, x.astype(np.float32))
