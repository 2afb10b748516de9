"""GPU parity of top-k sampling (exact top-k of the allowed scores, then the
Gumbel-max over the kept ids) against the CPU oracle.

Most cases give the oracle the logits the GPU computed (read back from the
unfused path's workspace), so the unfused path and the oracle select from
identical fp32 scores and differ only in the noise (fp32 on the GPU, fp64 in
the oracle), which the near-tie rule covers.  The fused path (k <= 64) sums its
scores in its own order and is held to the top-k reading of the rule (final
argmax or k-th boundary near ties); one group of cases compares it end to end
with the oracle's own logits.  Cases: tiny and ragged shapes,
k = 1 (plain argmax of the scores), k >= the allowed count (no-op), exact ties
across the k-th boundary (kept by lower id), masks, and boundaries wider than
the selection kernel's candidate buffer (refinement levels and the in-order
pass over equal keys).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_ids, check_ids_topk, dev_bf16, dev_words, oracle_p_fn, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch

    import lm_head_matmul_amd as fs_mod

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return fs_mod


@pytest.fixture(scope="module")
def ctx(fs):
    import torch

    c = fs.fs_create(0, max_B=256, max_V=262144, max_top_k=5000)
    torch.cuda.synchronize()
    yield c
    torch.cuda.synchronize()
    fs.fs_destroy(c)


def _gpu_logits(fs, ctx, Hd, Wd, B, V, path=0):
    import torch

    ws = torch.empty((B, (V + 3) // 4 * 4), dtype=torch.float32, device="cuda")
    fs.fs_unfused_sample(ctx, Hd, Wd, 1.0, 0, 0, logits_ws=ws, path=path)
    torch.cuda.synchronize()
    return np.ascontiguousarray(ws.cpu().numpy()[:, :V])


def _sample(fs, ctx, Hd, Wd, T, seed, steps, top_k, mask=None, path=0, unfused=False):
    import torch

    outs = []
    for s in steps:
        if unfused:
            outs.append(fs.fs_unfused_sample(ctx, Hd, Wd, T, seed, s, mask=mask, top_k=top_k, path=path))
        else:
            outs.append(fs.fs_fmms_sample(ctx, Hd, Wd, T, seed, s, mask=mask, top_k=top_k, path=path))
    torch.cuda.synchronize()
    return torch.stack(outs).cpu().numpy()


def _check(fs, ctx, H, W, T, seed, nsteps, top_k, mask_np=None, path=0, label=""):
    """The unfused path (stored logits, then selection) samples exactly what the oracle
    samples from the same stored logits; the fused path (for k <= 64: candidate lists, no
    stored logits, its scores summed in another fp32 order) agrees with it up to near ties
    of the final argmax or of the k-th boundary."""
    B, V = H.shape[0], W.shape[0]
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    md = None if mask_np is None else dev_words(mask_np)
    L = _gpu_logits(fs, ctx, Hd, Wd, B, V, path)
    fused = _sample(fs, ctx, Hd, Wd, T, seed, range(nsteps), top_k, md, path)
    unfused = _sample(fs, ctx, Hd, Wd, T, seed, range(nsteps), top_k, md, path, unfused=True)
    rows = np.arange(B)
    ora, _ = oracle.sample_rows_steps(L, rows, T, seed, 0, nsteps, mask=mask_np, top_k=top_k)
    n = check_ids(unfused, ora, oracle_p_fn(L, rows, T, seed, 0, mask=mask_np, top_k=top_k), label + " unfused")
    m = check_ids_topk(fused, ora, L, rows, T, seed, 0, top_k, mask=mask_np, label=label + " fused")
    say(f"{label}: near-tie mismatches {n} (unfused), {m} (fused) over {fused.size} draws")
    return fused, L


@pytest.mark.parametrize("B,d,V,T,k,path", [
    (4, 256, 4096, 1.0, 50, 0),
    (4, 256, 4096, 1.0, 50, 2),
    (8, 520, 3000, 0.7, 5, 0),
    (3, 256, 1000, 1.0, 1000, 0),   # k = V: every id kept
    (5, 264, 700, 1.3, 4999, 0),    # k > V
    (20, 1024, 5000, 0.8, 64, 0),
    (70, 264, 333, 1.0, 17, 0),     # more rows than one workspace chunk
])
def test_topk_parity(fs, ctx, B, d, V, T, k, path):
    say(f"top-k parity B={B} d={d} V={V} T={T} k={k} path={path}")
    H = synth.normal_bf16(B, d, seed=21)
    W = synth.normal_bf16(V, d, seed=22, std=0.05)
    _check(fs, ctx, H, W, T, 3, 20, k, path=path, label=f"topk k={k}")


@pytest.mark.parametrize("B,d,V,T,k", [
    (4, 256, 4096, 1.0, 50),
    (8, 520, 3000, 0.7, 5),
    (20, 1024, 5000, 0.8, 64),
    (33, 2048, 20011, 0.9, 50),
    (70, 264, 333, 1.0, 17),
])
def test_topk_end_to_end_vs_oracle_logits(fs, ctx, B, d, V, T, k):
    # end to end: the oracle computes its own logits from the same bf16 operands;
    # the kept sets may differ only at the k-th boundary, the draws only at near ties
    say(f"top-k end to end B={B} d={d} V={V} T={T} k={k}")
    H = synth.normal_bf16(B, d, seed=41)
    W = synth.normal_bf16(V, d, seed=42, std=0.05)
    L = oracle.logits(H, W)
    allowed = np.random.default_rng(43).random((B, V)) >= 0.25
    mask = synth.pack_mask(allowed)
    rows = np.arange(B)
    for mnp in (None, mask):
        md = None if mnp is None else dev_words(mnp)
        gpu = _sample(fs, ctx, dev_bf16(H), dev_bf16(W), T, 11, range(15), k, md)
        ora, _ = oracle.sample_rows_steps(L, rows, T, 11, 0, 15, mask=mnp, top_k=k)
        n = check_ids_topk(gpu, ora, L, rows, T, 11, 0, k, mask=mnp, label=f"top-k e2e k={k}")
        say(f"  mask={mnp is not None}: {n} near-tie mismatches over {gpu.size} draws")


def test_topk_one_is_argmax(fs, ctx):
    B, d, V = 6, 512, 2500
    H = synth.normal_bf16(B, d, seed=23)
    W = synth.normal_bf16(V, d, seed=24, std=0.05)
    ids, L = _check(fs, ctx, H, W, 1.0, 4, 10, 1, label="k=1")
    want = np.argmax(L, axis=1)  # numpy: first index of the maximum
    assert np.all(ids == want[None, :])


@pytest.mark.parametrize("V", [3000, 40000])  # one segment per row, several
def test_topk_ties_at_boundary(fs, ctx, V):
    # integer logits: many exactly equal scores, the k-th value falls inside a tie group
    B, d, k = 6, 256, 40
    H = synth.small_int_bf16(B, d, seed=25)
    W = synth.small_int_bf16(V, d, seed=26, lo=-1, hi=1)
    ids, L = _check(fs, ctx, H, W, 1.0, 5, 40, k, label="ties")
    for b in range(B):  # every draw is one of the k lowest-id ids among the top scores
        order = np.lexsort((np.arange(V), -L[b].astype(np.float64)))
        kept = set(order[:k].tolist())
        assert set(ids[:, b].tolist()) <= kept


def test_topk_with_mask(fs, ctx):
    B, d, V, k = 10, 520, 3000, 30
    H = synth.normal_bf16(B, d, seed=27)
    W = synth.outlier_bf16(V, d, 28, 29, 0.05, 0.5, 0.01)
    allowed = np.random.default_rng(30).random((B, V)) >= 0.3
    allowed[2] = False                   # nothing allowed: -1
    allowed[3] = False
    allowed[3, [5, 2999, 1400]] = True   # fewer allowed ids than k: all of them kept
    mask = synth.pack_mask(allowed)
    ids, _ = _check(fs, ctx, H, W, 1.0, 6, 20, k, mask_np=mask, label="masked top-k")
    assert np.all(ids[:, 2] == -1)
    assert set(ids[:, 3].tolist()) <= {5, 2999, 1400}
    for b in range(B):
        if b != 2:
            assert np.all(allowed[b, ids[:, b]])


@pytest.mark.parametrize("V", [9000, 40000])
def test_topk_all_scores_equal(fs, ctx, V):
    # every score is 0: the boundary holds all V equal keys (more than the
    # selection kernel gathers), so the k lowest ids are kept
    B, d, k = 3, 256, 25
    H = np.zeros((B, d), np.uint16)
    W = synth.normal_bf16(V, d, seed=31)
    ids, L = _check(fs, ctx, H, W, 1.0, 7, 30, k, label="all equal")
    assert np.all(L == 0)
    assert np.all((ids >= 0) & (ids < k))


@pytest.mark.parametrize("V", [12000, 40000])
def test_topk_narrow_score_range(fs, ctx, V):
    # scores within a few ulps of 1.0 for most ids: the first-level bin is too
    # wide for the candidate buffer and the selection refines it
    B, d, k = 2, 256, 50
    H = np.zeros((B, d), np.uint16)
    H[:, 0] = 0x3F80  # 1.0
    W = np.zeros((V, d), np.uint16)
    rng = np.random.default_rng(32)
    W[:, 0] = 0x3F80 + rng.integers(0, 8, V).astype(np.uint16)  # 1.0 .. 1.0546875
    W[::7, 0] = 0x3F00  # some far below (0.5)
    ids, L = _check(fs, ctx, H, W, 1.0, 8, 30, k, label="narrow range")
    for b in range(B):
        order = np.lexsort((np.arange(V), -L[b].astype(np.float64)))
        assert set(ids[:, b].tolist()) <= set(order[:k].tolist())


def test_topk_rows_held_by_one_segment(fs, ctx):
    # a full-size row is split into segments, each adding to the row's
    # histogram only its bins from its own k-th score up; masks that put all
    # of a row's allowed ids in one stretch of the vocabulary check the cases
    # where that cut matters: many, exactly k + 1, exactly k, and fewer than k
    # allowed ids in one segment, k spread thinly over all segments, no mask
    B, d, V, k = 6, 256, 40000, 50
    H = synth.normal_bf16(B, d, seed=33)
    W = synth.normal_bf16(V, d, seed=34, std=0.05)
    allowed = np.zeros((B, V), bool)
    allowed[0, 100:1100] = True
    allowed[1, 300:300 + k + 1] = True
    allowed[2, 39000:39000 + k] = True
    allowed[3, 20000:20000 + k - 1] = True
    allowed[4, ::V // k] = True
    allowed[5] = True
    mask = synth.pack_mask(allowed)
    ids, L = _check(fs, ctx, H, W, 1.0, 9, 30, k, mask_np=mask, label="one-segment rows")
    for b in range(B):
        s = np.where(allowed[b], L[b].astype(np.float64), -np.inf)
        order = np.lexsort((np.arange(V), -s))
        kept = set(order[:min(k, int(allowed[b].sum()))].tolist())
        assert set(ids[:, b].tolist()) <= kept, b
    assert len(set(ids[:, 3].tolist())) > 10  # all k - 1 allowed ids stay in play


@pytest.mark.parametrize("B,d,V,k,lo,n_hot", [
    (5, 256, 20000, 50, 5000, 100),    # the top 50 in one stretch: most lists of one tile saturate
    (3, 512, 151936, 64, 77777, 64),   # exactly k hot ids, a full-size vocabulary
    (4, 1024, 9000, 20, 0, 4),         # fewer hot ids than k at the start of the vocabulary
])
def test_topk_fused_rescoring(fs, ctx, B, d, V, k, lo, n_hot):
    # a block of consecutive "hot" ids scores far above the rest, so the row's
    # top k crowd into the lists of a few waves of one or two tiles; their bounds
    # then reach the k-th score and the merge rescores those tiles from H and W
    say(f"fused top-k rescoring B={B} d={d} V={V} k={k} hot ids [{lo}, {lo + n_hot})")
    H = synth.normal_bf16(B, d, seed=61)
    H[:, 0] = 0x3F80  # 1.0
    W = synth.normal_bf16(V, d, seed=62, std=0.05)
    W[:, 0] = 0
    W[lo:lo + n_hot, 0] = 0x4100  # 8.0
    L = oracle.logits(H, W)
    rows = np.arange(B)
    gpu = _sample(fs, ctx, dev_bf16(H), dev_bf16(W), 1.0, 12, range(20), k)
    ora, _ = oracle.sample_rows_steps(L, rows, 1.0, 12, 0, 20, top_k=k)
    n = check_ids_topk(gpu, ora, L, rows, 1.0, 12, 0, k, label="fused rescoring")
    say(f"  {n} near-tie mismatches over {gpu.size} draws")
    if n_hot >= k:
        assert np.all((gpu >= lo) & (gpu < lo + n_hot))
    # the draws follow the restricted softmax: every hot id of a row with n_hot <= k is drawn
    if n_hot < k:
        assert len(set(gpu[:, 0].tolist()) & set(range(lo, lo + n_hot))) >= 1


@pytest.mark.parametrize("B,d,V,T,k,top_p", [
    (4, 256, 4096, 1.0, 50, 0.9),
    (8, 520, 3000, 0.7, 20, 0.5),
    (20, 1024, 5000, 0.8, 64, 0.95),
    (33, 2048, 20011, 0.9, 50, 0.3),
    (3, 512, 2000, 1.0, 8, 1e-6),   # a tiny nucleus: the argmax of the scores
])
def test_top_p_end_to_end_vs_oracle_logits(fs, ctx, B, d, V, T, k, top_p):
    # top-k, then the nucleus holding top_p of the kept mass, end to end against the
    # oracle's own logits; with a mask as well
    say(f"top-p end to end B={B} d={d} V={V} T={T} k={k} top_p={top_p}")
    H = synth.normal_bf16(B, d, seed=71)
    W = synth.normal_bf16(V, d, seed=72, std=0.05)
    L = oracle.logits(H, W)
    allowed = np.random.default_rng(73).random((B, V)) >= 0.25
    mask = synth.pack_mask(allowed)
    rows = np.arange(B)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    import torch

    for mnp in (None, mask):
        md = None if mnp is None else dev_words(mnp)
        gpu = torch.stack([fs.fs_fmms_sample_top_p(ctx, Hd, Wd, T, 13, s, k, top_p, mask=md) for s in range(15)])
        torch.cuda.synchronize()
        gpu = gpu.cpu().numpy()
        ora, _ = oracle.sample_rows_steps(L, rows, T, 13, 0, 15, mask=mnp, top_k=k, top_p=top_p)
        n = check_ids_topk(gpu, ora, L, rows, T, 13, 0, k, mask=mnp, label=f"top-p {top_p}", top_p=top_p)
        say(f"  mask={mnp is not None}: {n} near-tie mismatches over {gpu.size} draws")
        if top_p < 1e-3:
            s = L.astype(np.float64) if mnp is None else np.where(synth.unpack_mask(mnp, V), L, -np.inf)
            assert np.all(gpu == np.argmax(s, axis=1)[None, :])


def test_top_p_one_equals_top_k(fs, ctx):
    import torch

    B, d, V, k = 6, 1024, 7000, 40
    Hd = dev_bf16(synth.normal_bf16(B, d, seed=74))
    Wd = dev_bf16(synth.normal_bf16(V, d, seed=75, std=0.05))
    a = torch.stack([fs.fs_fmms_sample(ctx, Hd, Wd, 0.9, 2, s, top_k=k) for s in range(10)])
    b = torch.stack([fs.fs_fmms_sample_top_p(ctx, Hd, Wd, 0.9, 2, s, k, 1.0) for s in range(10)])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_top_p_argument_checks(fs, ctx):
    import torch

    Hd = dev_bf16(synth.normal_bf16(2, 256, seed=76))
    Wd = dev_bf16(synth.normal_bf16(500, 256, seed=77, std=0.05))
    out = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    for k, tp, path, code in ((0, 0.5, 0, -1), (65, 0.5, 0, -2), (10, 0.0, 0, -1), (10, 1.5, 0, -1),
                              (10, float("nan"), 0, -1), (10, 0.5, 1, -2), (5001, 0.5, 0, -3)):
        with pytest.raises(fs.FSError) as ei:
            fs.fs_fmms_sample_top_p(ctx, Hd, Wd, 1.0, 0, 0, k, tp, out=out, path=path)
        assert ei.value.code == code, (k, tp, path)
    torch.cuda.synchronize()
    assert torch.all(out == -7).item()
