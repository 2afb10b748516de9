"""Pins of the oracle's sampler against what the method fixes.

  * Gumbel-Max: argmax of logits/T plus i.i.d. standard Gumbel noise is an
    exact draw from softmax(logits/T) [readus.org FlashSampling summary,
    section "Gumbel Max Trick" (Theorem 2.1); arXiv 2603.15854 abstract].
    Checked by chi-square over 10^6 draws at V = 16.
  * argmax decomposes over any partition of the vocabulary [abstract]:
    combined tile maxima equal the global argmax bit for bit.
  * masked ids are never drawn; top-k keeps an exact candidate set and samples
    inside it [readus.org summary, section on Top-K and masking].
  * grouped sampling equals flat sampling in distribution (hierarchical
    factorization [abstract]; group log-sum-exp "captains" [readus.org summary,
    section "Group Gumbel Max"]), and the max-combine equals flat exactly.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import chi2 as chi2_dist

import oracle
import synth

P_MIN = 1e-3


def chi2_p(counts, probs):
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    keep = probs > 0
    assert counts[~keep].sum() == 0, "draws landed on zero-probability ids"
    if keep.sum() == 1:
        return 1.0
    exp = n * probs[keep]
    stat = float(((counts[keep] - exp) ** 2 / exp).sum())
    return chi2_dist.sf(stat, keep.sum() - 1)


@pytest.fixture(scope="module")
def tiny_v16():
    # The tiny workload's V = 16 variant: B = 4, d = 256, H ~ N(0,1), W ~ N(0, 1/d).
    H = synth.workload_H("tiny")
    W = synth.normal_bf16(16, 256, seed=2, std=1 / 16)
    return oracle.logits(H, W)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_gumbel_max_matches_softmax_chi2(tiny_v16, T):
    L = tiny_v16
    draws = oracle.sample_steps(L, T, seed=0, step0=0, nsteps=1_000_000)
    for b in range(L.shape[0]):
        probs = softmax(L[b].astype(np.float64) / np.float64(np.float32(T)))
        counts = np.bincount(draws[:, b], minlength=16)
        assert chi2_p(counts, probs) > P_MIN, (b, T)


def test_chi2_detects_a_planted_temperature_mistake(tiny_v16):
    # Sanity of the statistic: draws at T = 0.7 are far from softmax(logits / 1.0).
    L = tiny_v16
    draws = oracle.sample_steps(L, 0.7, seed=0, step0=0, nsteps=200_000)
    probs = softmax(L[0].astype(np.float64))
    assert chi2_p(np.bincount(draws[:, 0], minlength=16), probs) < 1e-12


def test_partition_invariance_bitwise():
    rng = np.random.default_rng(1)
    H = synth.normal_bf16(3, 64, seed=11)
    W = synth.normal_bf16(997, 64, seed=12, std=0.2)
    L = oracle.logits(H, W)
    for step in range(6):
        flat = oracle.sample_from_logits(L, 1.0, seed=5, step=step)
        for trial in range(5):
            n_cut = int(rng.integers(1, 60))
            cuts = np.sort(rng.choice(np.arange(1, 997), n_cut, replace=False))
            bounds = np.concatenate([[0], cuts, [997]]).astype(np.int64)
            tmax, targ = oracle.tile_maxima(L, 1.0, 5, step, bounds)
            for b in range(3):
                best = int(np.argmax(tmax[b]))  # first maximal tile = lowest ids
                assert targ[b, best] == flat[b]


def test_argmax_tie_rule():
    p = np.array([1.0, 3.0, 2.0, 3.0, -np.inf], np.float32)
    assert oracle.argmax(p) == 1
    assert oracle.argmax(np.full(5, -np.inf, np.float32)) == -1
    assert oracle.argmax(np.array([np.nan, 0.5, np.nan], np.float32)) == 1


def test_mask_never_drawn_and_restricted_softmax():
    H = synth.workload_H("tiny")
    W = synth.normal_bf16(16, 256, seed=2, std=1 / 16)
    L = oracle.logits(H, W)
    allowed = np.ones((4, 16), bool)
    allowed[0, [0, 3, 5]] = False
    allowed[1, ::2] = False
    allowed[2, 1:] = False
    mask = synth.pack_mask(allowed)
    draws = oracle.sample_steps(L, 1.0, seed=9, step0=0, nsteps=300_000, mask=mask)
    for b in range(4):
        assert np.all(allowed[b, draws[:, b]])
        logit = np.where(allowed[b], L[b].astype(np.float64), -np.inf)
        assert chi2_p(np.bincount(draws[:, b], minlength=16), softmax(logit)) > P_MIN


def test_all_masked_row_gives_minus_one():
    L = np.zeros((2, 40), np.float32)
    allowed = np.ones((2, 40), bool)
    allowed[1] = False
    out = oracle.sample_from_logits(L, 1.0, 0, 0, mask=synth.pack_mask(allowed))
    assert out[1] == -1 and 0 <= out[0] < 40


def test_mask_word_layout():
    # bit (v & 31) of word (v >> 5), 1 = allowed
    allowed = np.zeros((1, 70), bool)
    allowed[0, [0, 31, 32, 69]] = True
    w = synth.pack_mask(allowed)
    assert w.shape == (1, 3)
    assert w[0, 0] == (1 | (1 << 31)) and w[0, 1] == 1 and w[0, 2] == (1 << 5)
    assert np.array_equal(synth.unpack_mask(w, 70), allowed)


def test_top_k_set_matches_sort():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(5000).astype(np.float32)
    x[100:110] = x[50]  # ties around whatever value x[50] has
    for k in [1, 5, 50, 4999, 5000, 6000]:
        s = oracle.scores_row(x, 0.7, top_k=k)
        ref_s = (x / np.float32(0.7)).astype(np.float32)
        order = np.lexsort((np.arange(5000), -ref_s))  # score desc, id asc
        keep = np.zeros(5000, bool)
        keep[order[: min(k, 5000)]] = True
        assert np.array_equal(np.isfinite(s), keep), k
        assert np.array_equal(s[keep], ref_s[keep])


def test_top_k_boundary_ties_keep_lower_ids():
    x = np.array([5, 1, 3, 3, 3, 0, 3], np.float32)
    s = oracle.scores_row(x, 1.0, top_k=3)
    assert np.array_equal(np.isfinite(s), [True, False, True, True, False, False, False])


def test_top_k_applies_after_mask():
    x = np.array([9, 8, 7, 6, 5], np.float32)
    allowed = np.array([[False, True, True, True, True]])
    s = oracle.scores_row(x, 1.0, mask_row=synth.pack_mask(allowed)[0], top_k=2)
    assert np.array_equal(np.isfinite(s), [False, True, True, False, False])


def test_top_k_draws_match_restricted_softmax(tiny_v16):
    L = tiny_v16
    k = 5
    draws = oracle.sample_steps(L, 0.7, seed=3, step0=0, nsteps=300_000, top_k=k)
    for b in range(4):
        s = L[b] / np.float32(0.7)
        order = np.lexsort((np.arange(16), -s))
        probs = np.zeros(16)
        probs[order[:k]] = softmax(s[order[:k]].astype(np.float64))
        assert chi2_p(np.bincount(draws[:, b], minlength=16), probs) > P_MIN


def test_group_max_combine_equals_flat_bitwise():
    rng = np.random.default_rng(8)
    H = synth.normal_bf16(4, 64, seed=13)
    W = synth.normal_bf16(512, 64, seed=14, std=0.3)
    L = oracle.logits(H, W)
    for trial in range(4):
        cuts = np.sort(rng.choice(np.arange(1, 512), 7, replace=False))
        bounds = np.concatenate([[0], cuts, [512]]).astype(np.int64)
        g = oracle.grouped_sample_steps(L, 1.0, 2, 0, 50, bounds, oracle.GROUP_MODE_MAX)
        f = oracle.sample_steps(L, 1.0, 2, 0, 50)
        assert np.array_equal(g, f)


def test_group_summary_pieces_match_direct_definition():
    H = synth.normal_bf16(3, 64, seed=15)
    W = synth.normal_bf16(256, 64, seed=16, std=0.3)
    L = oracle.logits(H, W)
    allowed = np.random.default_rng(1).random((3, 256)) > 0.3
    mask = synth.pack_mask(allowed)
    lse, pmax, arg = oracle.group_summary(L, 64, 64, 0.7, seed=4, step=2, mask=mask)
    for b in range(3):
        s = (L[b] / np.float32(0.7)).astype(np.float32)
        sel = np.arange(64, 128)
        ok = allowed[b, sel]
        ref_lse = logsumexp(s[sel][ok].astype(np.float64))
        assert abs(lse[b] - ref_lse) <= 1e-6 * max(1, abs(ref_lse))
        p = oracle.perturbed_row(L[b], 0.7, 4, 2, b, mask_row=mask[b])
        assert pmax[b] == p[64:128].max()
        assert arg[b] == 64 + int(np.argmax(p[64:128]))


def _contiguous_partitions(V):
    for m in range(1 << (V - 1)):
        cuts = [i + 1 for i in range(V - 1) if (m >> i) & 1]
        yield np.array([0, *cuts, V], np.int64)


@pytest.mark.slow
def test_grouped_gumbel_equals_flat_in_distribution_all_partitions():
    # Every contiguous partition of V = 8 ids (128 of them): the hierarchical sampler's
    # draws follow softmax(logits).  Bonferroni-corrected threshold over the partitions.
    H = synth.normal_bf16(1, 64, seed=17)
    W = synth.normal_bf16(8, 64, seed=18, std=0.15)
    L = oracle.logits(H, W)
    probs = softmax(L[0].astype(np.float64))
    parts = list(_contiguous_partitions(8))
    pvals = []
    for i, bounds in enumerate(parts):
        draws = oracle.grouped_sample_steps(L, 1.0, 100 + i, 0, 40_000, bounds, oracle.GROUP_MODE_GUMBEL)
        pvals.append(chi2_p(np.bincount(draws[:, 0], minlength=8), probs))
    assert min(pvals) > P_MIN / len(parts)


def test_grouped_gumbel_group_choice_follows_softmax_of_lse():
    # P(group k) = softmax(lse)_k: check the group of each draw at a larger V.
    H = synth.normal_bf16(2, 64, seed=19)
    W = synth.normal_bf16(64, 64, seed=20, std=0.2)
    L = oracle.logits(H, W)
    bounds = synth.group_bounds(64, 8)
    draws = oracle.grouped_sample_steps(L, 1.0, 3, 0, 200_000, bounds, oracle.GROUP_MODE_GUMBEL)
    for b in range(2):
        lse = np.array([logsumexp(L[b, bounds[k]:bounds[k + 1]].astype(np.float64)) for k in range(8)])
        counts = np.bincount(draws[:, b] // 8, minlength=8)
        assert chi2_p(counts, softmax(lse)) > P_MIN
        assert chi2_p(np.bincount(draws[:, b], minlength=64), softmax(L[b].astype(np.float64))) > P_MIN


def test_group_combine_rejects_empty_groups():
    lse = np.array([[-np.inf], [0.0]], np.float32)
    pmax = np.array([[-np.inf], [1.0]], np.float32)
    arg = np.array([[-1], [7]], np.int32)
    for mode in (oracle.GROUP_MODE_GUMBEL, oracle.GROUP_MODE_MAX):
        assert oracle.group_combine(lse, pmax, arg, 0, 0, mode)[0] == 7
    lse[1] = -np.inf
    pmax[1] = -np.inf
    arg[1] = -1
    assert oracle.group_combine(lse, pmax, arg, 0, 0, oracle.GROUP_MODE_GUMBEL)[0] == -1


def test_max_stability_of_group_maxima():
    # max_v (s_v + g_v) over a group is Gumbel(lse, 1): pmax - lse has mean gamma and variance pi^2/6.
    H = synth.normal_bf16(1, 64, seed=21)
    W = synth.normal_bf16(48, 64, seed=22, std=0.25)
    L = oracle.logits(H, W)
    diffs = []
    for step in range(20000):
        lse, pmax, _ = oracle.group_summary(L, 0, 48, 1.0, seed=6, step=step)
        diffs.append(float(pmax[0]) - float(lse[0]))
    diffs = np.array(diffs)
    assert abs(diffs.mean() - 0.5772156649) < 0.03
    assert abs(diffs.var() - math.pi**2 / 6) < 0.08


def test_end_to_end_equals_logits_then_sample():
    H = synth.workload_H("tiny")
    W = synth.workload_W("tiny")
    a = oracle.fmms_sample(H, W, 1.0, 0, 0)
    b = oracle.sample_from_logits(oracle.logits(H, W), 1.0, 0, 0)
    assert np.array_equal(a, b)
    assert np.all((a >= 0) & (a < 4096))
