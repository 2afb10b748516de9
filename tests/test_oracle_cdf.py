"""Pins of the oracle's conventional comparator: softmax, prefix sum and an
inverse-CDF search with one uniform per row and step (reading R9).  This is
the pipeline the fused sampler replaces [readus.org FlashSampling summary, the
essay part on the softmax pipeline]; it is a baseline, not the method.

  * closed form: with scores ln 1 .. ln 4 the probabilities are k / 10, so the
    draw is the interval of the cumulative (0.1, 0.3, 0.6, 1.0) that holds u;
  * chi-square against softmax(logits / T) at V = 16;
  * the uniforms are uniform on (0, 1) and come from their own Philox counter
    range;
  * masked ids are never drawn, a lone allowed id always is, none gives -1.
"""
import numpy as np
from scipy.special import softmax
from scipy.stats import kstest

import oracle
import synth
from test_oracle_sampling import P_MIN, chi2_p


def test_closed_form_quarters():
    L = np.log(np.array([[1.0, 2.0, 3.0, 4.0]], np.float32))
    ids, u = oracle.cdf_sample_rows_steps(L, np.array([0]), 1.0, 3, 0, 20_000)
    bounds = np.array([0.1, 0.3, 0.6])
    want = np.searchsorted(bounds, u[:, 0], side="right")  # interval of u in the cumulative
    near = np.min(np.abs(u[:, 0][:, None] - bounds[None, :]), axis=1) < 1e-6
    assert np.array_equal(ids[~near, 0], want[~near])
    assert np.bincount(ids[:, 0], minlength=4).min() > 1000


def test_matches_softmax_chi2():
    H = synth.workload_H("tiny")
    W = synth.normal_bf16(16, 256, seed=2, std=1 / 16)
    L = oracle.logits(H, W)
    for T in (1.0, 0.7):
        ids, _ = oracle.cdf_sample_rows_steps(L, np.arange(L.shape[0]), T, 0, 0, 200_000)
        for b in range(L.shape[0]):
            probs = softmax(L[b].astype(np.float64) / np.float64(np.float32(T)))
            assert chi2_p(np.bincount(ids[:, b], minlength=16), probs) > P_MIN, (b, T)


def test_uniforms_are_uniform_and_inside_the_open_interval():
    _, u = oracle.cdf_sample_rows_steps(np.zeros((3, 2), np.float32), np.array([0, 1, 7]), 1.0, 9, 0, 40_000)
    assert kstest(u.ravel(), "uniform").pvalue > P_MIN
    assert oracle.uniform64(0) == 1.0 / 4294967297.0
    assert 0.0 < oracle.uniform64(0) and oracle.uniform64(2**32 - 1) < 1.0


def test_uniform_counter_range_is_its_own():
    # word 0 of Philox at counter (0x80000000, row, step): disjoint from the
    # vocabulary's (v >> 2 < 2^29) and the group noise's (0x40000000 | k) words
    for seed, step, row in [(0, 0, 0), (5, 7, 3), (2**40 + 1, 2**33 + 5, 11)]:
        key = [seed & 0xFFFFFFFF, seed >> 32]
        ctr = [0x80000000, row, step & 0xFFFFFFFF, step >> 32]
        assert oracle.uniform_bits(seed, step, row) == oracle.philox4x32_10(key, ctr)[0]
    assert 0x80000000 > (2**31 >> 2) and 0x80000000 > (0x40000000 | 4095)


def test_mask_cases():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((3, 70)).astype(np.float32)
    allowed = rng.random((3, 70)) > 0.5
    allowed[1] = False
    allowed[1, 33] = True
    allowed[2] = False
    mask = synth.pack_mask(allowed)
    ids, _ = oracle.cdf_sample_rows_steps(L, np.arange(3), 1.0, 1, 0, 3000, mask=mask)
    assert np.all(allowed[0, ids[:, 0]])
    assert np.all(ids[:, 1] == 33)
    assert np.all(ids[:, 2] == -1)
