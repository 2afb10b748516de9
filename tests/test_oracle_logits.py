"""Pins of the oracle's LM-head product logits = H W^T.

The fused sampler computes the LM-head logits tile by tile on chip
[FlashSampling, arXiv 2603.15854, abstract].  The oracle sums the exact bf16
products in fp64 and rounds once to fp32.  Checked here against exact
rational arithmetic, exact integer sums, numpy's fp64 matmul, and (for the
fp32-accumulated variant the kernels mirror) Higham's bound on recursive
summation error (Higham, Accuracy and Stability of Numerical Algorithms, ch. 3).
"""
from fractions import Fraction

import numpy as np

import oracle
import synth


def test_logits_exact_rationals():
    # A few entries against the definition in exact rational arithmetic: bf16 values are
    # dyadic rationals, so sum_k H[b,k] W[v,k] is exact; fp32 rounding of it must match.
    H = synth.normal_bf16(3, 96, seed=1)
    W = synth.normal_bf16(37, 96, seed=2, std=0.05)
    L = oracle.logits(H, W)
    Hf = synth.bf16_to_f32(H).astype(np.float64)
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    for b in range(3):
        for v in [0, 1, 17, 36]:
            exact = sum(Fraction(float(Hf[b, k])) * Fraction(float(Wf[v, k])) for k in range(96))
            assert np.float32(float(exact)) == L[b, v], (b, v)
    assert L.shape == (3, 37)  # rows are H rows, columns are W rows (no transposed operand)


def test_logits_integer_inputs_exact():
    H = synth.small_int_bf16(5, 256, seed=3)
    W = synth.small_int_bf16(300, 256, seed=4)
    L = oracle.logits(H, W)
    ref = synth.bf16_to_f32(H).astype(np.int64) @ synth.bf16_to_f32(W).astype(np.int64).T
    assert np.array_equal(L.astype(np.int64), ref)
    # fp32 accumulation is exact here too (|partial sums| < 2^24)
    assert np.array_equal(oracle.logits(H, W, fp32_acc=True), L)


def test_logits_vs_numpy_fp64_matmul():
    H = synth.normal_bf16(4, 512, seed=5)
    W = synth.normal_bf16(1000, 512, seed=6, std=0.02)
    L = oracle.logits(H, W)
    ref = (synth.bf16_to_f32(H).astype(np.float64) @ synth.bf16_to_f32(W).astype(np.float64).T).astype(np.float32)
    ulp = np.abs(L.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    assert (ulp == 0).mean() > 0.999


def test_fp32_accumulation_within_higham_bound():
    d = 4096
    H = synth.normal_bf16(2, d, seed=7)
    W = synth.normal_bf16(500, d, seed=8, std=0.02)
    L32 = oracle.logits(H, W, fp32_acc=True).astype(np.float64)
    Hf = synth.bf16_to_f32(H).astype(np.float64)
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    exact = Hf @ Wf.T
    absum = np.abs(Hf) @ np.abs(Wf).T
    u = 2.0**-24
    gamma = d * u / (1 - d * u)
    assert np.all(np.abs(L32 - exact) <= gamma * absum + 1e-30)


def test_logits_respects_leading_dimension():
    # ldh/ldw larger than d: the oracle must read only the first d entries of each row.
    H = synth.normal_bf16(2, 64, seed=9)
    W = synth.normal_bf16(10, 64, seed=10)
    Hp = np.zeros((2, 80), np.uint16)
    Wp = np.zeros((10, 72), np.uint16)
    Hp[:, :64] = H
    Wp[:, :64] = W
    Hp[:, 64:] = synth.bf16_round(np.full((2, 16), 1e3, np.float32))
    Wp[:, 64:] = synth.bf16_round(np.full((10, 8), 1e3, np.float32))
    out = np.empty((2, 10), np.float32)
    oracle.lib().fso_logits(Hp.ctypes.data, 80, Wp.ctypes.data, 72, 2, 64, 10, out.ctypes.data)
    assert np.array_equal(out, oracle.logits(H, W))
