"""GPU parity of the conventional comparator (softmax, prefix sum, inverse-CDF
search), which the fused sampler is measured against.

The oracle is given the logits the GPU computed (read back from the unfused
path's workspace; the comparator's logits pass is the same kernel), so both
sides sample from identical fp32 scores.  The GPU works in fp32: exp with
relative error near 1e-6 and running sums over up to 151936 terms in sequential
runs of a few dozen and trees of depth 15, so its cumulative sums are within a
few 1e-6 of the total of the oracle's fp64 ones.  A drawn id may differ from the
oracle's only if u times the total lies within CDF_TOL of the total from the
GPU id's interval of the oracle's cumulative sum, and ids agree on at least
99.9% of draws.  The probabilities left in the workspace match the oracle's
softmax to PROB_RTOL.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import ID_MATCH_MIN, dev_bf16, dev_words, say

pytestmark = pytest.mark.gpu

CDF_TOL = 1e-4
PROB_RTOL = 1e-4


@pytest.fixture(scope="module")
def fs():
    import torch

    import lm_head_matmul_amd as fs_mod

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return fs_mod


@pytest.fixture(scope="module")
def ctx(fs):
    import torch

    c = fs.fs_create(0, max_B=128, max_V=262144, max_top_k=0)
    torch.cuda.synchronize()
    yield c
    torch.cuda.synchronize()
    fs.fs_destroy(c)


def _weights(L_row, T, mask_row):
    s = oracle.scores_row(L_row, T, mask_row=mask_row).astype(np.float64)
    ok = np.isfinite(s)
    w = np.zeros_like(s)
    if ok.any():
        w[ok] = np.exp(s[ok] - s[ok].max())
    return w


def _check(fs, ctx, H, W, T, seed, nsteps, mask_np=None, label=""):
    import torch

    B, V = H.shape[0], W.shape[0]
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    md = None if mask_np is None else dev_words(mask_np)
    ldl = (V + 3) // 4 * 4
    ws = torch.empty((B, ldl), dtype=torch.float32, device="cuda")
    fs.fs_unfused_sample(ctx, Hd, Wd, 1.0, 0, 0, logits_ws=ws)
    torch.cuda.synchronize()
    L = np.ascontiguousarray(ws.cpu().numpy()[:, :V])
    got = []
    for t in range(nsteps):
        got.append(fs.fs_softmax_sample(ctx, Hd, Wd, T, seed, t, mask=md, logits_ws=ws))
    torch.cuda.synchronize()
    got = torch.stack(got).cpu().numpy()
    probs = ws.cpu().numpy()[:, :V]
    rows = np.arange(B)
    want, u = oracle.cdf_sample_rows_steps(L, rows, T, seed, 0, nsteps, mask=mask_np)
    mism = 0
    for b in range(B):
        w = _weights(L[b], T, None if mask_np is None else mask_np[b])
        Z = w.sum()
        if Z == 0:
            assert np.all(got[:, b] == -1), f"{label}: row {b} has no allowed id"
            assert np.all(probs[b] == 0)
            continue
        p_ref = w / Z
        assert np.allclose(probs[b], p_ref, rtol=PROB_RTOL, atol=1e-12), f"{label}: row {b} probabilities"
        C = np.concatenate([[0.0], np.cumsum(w)])
        for t in np.nonzero(got[:, b] != want[:, b])[0]:
            j = int(got[t, b])
            assert 0 <= j < V and w[j] > 0, f"{label}: step {t} row {b}: GPU id {j} has no mass"
            target = u[t, b] * Z
            assert C[j] - CDF_TOL * Z <= target <= C[j + 1] + CDF_TOL * Z, \
                f"{label}: step {t} row {b}: GPU {j} vs oracle {want[t, b]}, u={u[t, b]}"
            mism += 1
    assert 1.0 - mism / got.size >= ID_MATCH_MIN, f"{label}: {mism} mismatches over {got.size}"
    say(f"{label}: {mism} boundary mismatches over {got.size} draws")
    return got


@pytest.mark.parametrize("B,d,V,T", [
    (4, 256, 4096, 1.0),
    (8, 520, 3000, 0.7),
    (70, 264, 333, 1.0),
    (3, 512, 151936, 0.7),   # full vocabulary: many segments per row
    (1, 256, 5, 1.3),        # fewer ids than a quad
])
def test_softmax_comparator_parity(fs, ctx, B, d, V, T):
    say(f"comparator parity B={B} d={d} V={V} T={T}")
    H = synth.normal_bf16(B, d, seed=81)
    W = synth.normal_bf16(V, d, seed=82, std=2.0 / np.sqrt(d))
    _check(fs, ctx, H, W, T, 7, 30, label=f"comparator {B}x{V}")


def test_softmax_comparator_masks(fs, ctx):
    B, d, V = 6, 520, 3000
    H = synth.normal_bf16(B, d, seed=83)
    W = synth.outlier_bf16(V, d, 84, 85, 0.05, 0.5, 0.01)
    allowed = np.random.default_rng(86).random((B, V)) >= 0.3
    allowed[1] = False                # nothing allowed: -1
    allowed[4] = False
    allowed[4, 2222] = True           # a single allowed id: always drawn
    mask = synth.pack_mask(allowed)
    got = _check(fs, ctx, H, W, 1.0, 8, 30, mask_np=mask, label="masked comparator")
    assert np.all(got[:, 4] == 2222)
    for b in (0, 2, 3, 5):
        assert np.all(allowed[b, got[:, b]])


def test_softmax_comparator_draw_frequencies(fs, ctx):
    # row 0 is peaked (logit 10 at id 10, 0 elsewhere), row 1 is flat (all 0)
    import torch
    from scipy.stats import chisquare

    V, d, n = 64, 256, 4000
    H = np.zeros((2, d), np.uint16)
    H[0, 0] = 0x3F80  # 1.0
    W = np.zeros((V, d), np.uint16)
    W[10, 0] = 0x4120  # 10.0
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    ws = torch.empty((2, V), dtype=torch.float32, device="cuda")
    draws = torch.stack([fs.fs_softmax_sample(ctx, Hd, Wd, 1.0, 1, t, logits_ws=ws) for t in range(n)])
    torch.cuda.synchronize()
    draws = draws.cpu().numpy()
    p10 = np.exp(10.0) / (np.exp(10.0) + V - 1)
    frac = np.mean(draws[:, 0] == 10)
    assert abs(frac - p10) < 5 * np.sqrt(p10 * (1 - p10) / n)
    assert chisquare(np.bincount(draws[:, 1], minlength=V)).pvalue > 1e-3
