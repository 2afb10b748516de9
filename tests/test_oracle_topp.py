"""Pins of the oracle's top-p (nucleus) filter, which follows top-k.

Two pages call the method compatible with nucleus (top-p) sampling without
giving a method [cjcn.com.cn and news.neo-ai.one FlashSampling articles].  The
oracle takes the published definition of nucleus sampling (Holtzman et al.,
"The Curious Case of Neural Text Degeneration", ICLR 2020) over the ids top-k
keeps: sorted by score (lower id first among equal scores), an id stays while
the mass of the ids before it is below top_p of the kept mass.  Pinned here by
  * a worked example whose nucleus follows from closed-form masses,
  * equal scores, where the nucleus is the lowest ids by a count,
  * the limits: top_p = 1 is top-k alone; a tiny top_p is the argmax of s,
  * chi-square of the draws against the softmax restricted to the nucleus,
  * the nucleus never leaving the top-k set and growing with top_p.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chi2 as chi2_dist

import oracle
import synth

P_MIN = 1e-3


def kept(L_row, T=1.0, top_k=0, top_p=1.0, mask_row=None):
    s = oracle.scores_row(np.asarray(L_row, np.float32), T, mask_row=mask_row, top_k=top_k, top_p=top_p)
    return set(np.flatnonzero(np.isfinite(s)).tolist())


def test_worked_example_closed_form():
    # scores 2, 1, 0, -1: masses e^2, e^1, e^0, e^-1 over Z; cumulative shares
    # 0.6439, 0.8808, 0.9680, 1 -- the nucleus holds one more id for every share below top_p
    Z = math.e ** 2 + math.e + 1.0 + 1.0 / math.e
    shares = [math.e ** 2 / Z, (math.e ** 2 + math.e) / Z, (math.e ** 2 + math.e + 1.0) / Z]
    assert abs(shares[0] - 0.6439) < 1e-4 and abs(shares[1] - 0.8808) < 1e-4 and abs(shares[2] - 0.9680) < 1e-4
    L = [2.0, 1.0, 0.0, -1.0]
    for p, size in [(0.3, 1), (0.6, 1), (0.65, 2), (0.8, 2), (0.9, 3), (0.96, 3), (0.97, 4), (1.0, 4)]:
        assert size == 1 + sum(c < p for c in shares)
        assert kept(L, top_p=p) == set(range(size)), p
    # the same row shuffled: the nucleus follows the scores, not the positions
    perm = [3, 0, 2, 1]
    Lp = [L[i] for i in perm]  # ids 0..3 carry scores -1, 2, 0, 1
    assert kept(Lp, top_p=0.8) == {1, 3}
    assert kept(Lp, top_p=0.9) == {1, 3, 2}


def test_equal_scores_keep_the_lowest_ids():
    # eight equal scores: each holds 1/8 of the mass, so top_p = 3/8 + tiny keeps
    # four ids (the mass before the fourth, 3/8, is below top_p) -- the four lowest
    L = np.zeros(8, np.float32)
    assert kept(L, top_p=0.376) == {0, 1, 2, 3}
    assert kept(L, top_p=0.375) == {0, 1, 2}  # 3/8 is exact in binary: not below top_p
    assert kept(L, top_p=1.0) == set(range(8))


def test_limits_top_p_one_and_tiny():
    H = synth.normal_bf16(5, 128, seed=31)
    W = synth.normal_bf16(700, 128, seed=32, std=0.15)
    L = oracle.logits(H, W)
    steps = 300
    a = oracle.sample_steps(L, 0.8, seed=3, step0=0, nsteps=steps, top_k=40)
    b = oracle.sample_steps(L, 0.8, seed=3, step0=0, nsteps=steps, top_k=40, top_p=1.0)
    assert np.array_equal(a, b)
    greedy = oracle.sample_steps(L, 0.8, seed=3, step0=0, nsteps=steps, top_k=40, top_p=1e-7)
    assert np.all(greedy == np.argmax(L, axis=1)[None, :])


def test_nucleus_inside_top_k_and_monotone():
    rng = np.random.default_rng(33)
    for trial in range(20):
        L = rng.normal(0, 2.0, 300).astype(np.float32)
        k = int(rng.integers(1, 60))
        top = kept(L, top_k=k)
        prev = set()
        for p in np.linspace(0.05, 1.0, 12):
            cur = kept(L, top_k=k, top_p=float(p))
            assert cur <= top and prev <= cur and len(cur) >= 1
            prev = cur
        assert prev == top


def _nucleus_probs(L_row, T, top_k, top_p, mask_row=None):
    """The restricted softmax: zero outside the oracle's kept set, renormalized inside."""
    s = L_row.astype(np.float64) / np.float64(np.float32(T))
    keep = np.zeros(s.shape, bool)
    keep[list(kept(L_row, T, top_k, top_p, mask_row))] = True
    probs = np.where(keep, softmax(np.where(keep, s, -np.inf)), 0.0)
    return probs


def chi2_p(counts, probs):
    counts = np.asarray(counts, np.float64)
    keep = probs > 0
    assert counts[~keep].sum() == 0, "draws landed outside the nucleus"
    if keep.sum() == 1:
        return 1.0
    exp = counts.sum() * probs[keep]
    return chi2_dist.sf(float(((counts[keep] - exp) ** 2 / exp).sum()), keep.sum() - 1)


@pytest.mark.slow
@pytest.mark.parametrize("top_k,top_p,T", [(16, 0.5, 1.0), (16, 0.9, 0.7), (6, 0.8, 1.0)])
def test_draws_follow_the_nucleus_softmax_chi2(top_k, top_p, T):
    H = synth.workload_H("tiny")
    W = synth.normal_bf16(16, 256, seed=2, std=1 / 16)
    L = oracle.logits(H, W)
    draws = oracle.sample_steps(L, T, seed=0, step0=0, nsteps=200_000, top_k=top_k, top_p=top_p)
    for b in range(L.shape[0]):
        probs = _nucleus_probs(L[b], T, top_k, top_p)
        assert (probs > 0).sum() >= 1
        assert chi2_p(np.bincount(draws[:, b], minlength=16), probs) > P_MIN, (b, top_k, top_p)


def test_mask_then_top_k_then_top_p():
    rng = np.random.default_rng(34)
    B, V = 3, 64
    L = rng.normal(0, 1.5, (B, V)).astype(np.float32)
    allowed = rng.random((B, V)) >= 0.4
    mask = synth.pack_mask(allowed)
    draws = oracle.sample_steps(L, 1.0, seed=9, step0=0, nsteps=60_000, mask=mask, top_k=12, top_p=0.75)
    for b in range(B):
        probs = _nucleus_probs(L[b], 1.0, 12, 0.75, mask[b])
        assert np.all(allowed[b][probs > 0])
        assert chi2_p(np.bincount(draws[:, b], minlength=V), probs) > P_MIN, b


def test_chi2_detects_a_planted_nucleus_mistake():
    # sanity of the statistic: draws from the 0.5-nucleus are far from the 0.9-nucleus softmax
    H = synth.workload_H("tiny")
    W = synth.normal_bf16(16, 256, seed=2, std=1 / 16)
    L = oracle.logits(H, W)
    draws = oracle.sample_steps(L, 1.0, seed=0, step0=0, nsteps=100_000, top_k=16, top_p=0.5)
    wrong = _nucleus_probs(L[0], 1.0, 16, 0.9)
    counts = np.bincount(draws[:, 0], minlength=16)
    exp = counts.sum() * wrong[wrong > 0]
    stat = float(((counts[wrong > 0] - exp) ** 2 / exp).sum())
    assert chi2_dist.sf(stat, (wrong > 0).sum() - 1) < 1e-12
