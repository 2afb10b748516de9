"""Helpers shared by the GPU parity tests (device transfer, the id parity rule)."""
import numpy as np
import torch

import oracle

# Sampled ids must agree with the oracle on >= 99.9% of rows; any mismatch must be a
# near-tie: the oracle's perturbed scores of the two ids differ by < 1e-3 (1 + |max|).
ID_MATCH_MIN = 0.999
NEAR_TIE_REL = 1e-3
# Per-tile maxima agree within 1e-3 relative (bf16 inputs, fp32 accumulation).
TILE_REL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_words(m: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint32).view(np.int32)).cuda()


def check_ids(gpu_ids, ora_ids, p_row, label=""):
    """gpu_ids, ora_ids: [S, R].  p_row(s, r) -> oracle perturbed scores of that row at that step.

    Returns the number of (near-tie) mismatches; fails on any other disagreement.
    """
    gpu_ids = np.asarray(gpu_ids)
    ora_ids = np.asarray(ora_ids)
    assert gpu_ids.shape == ora_ids.shape
    mism = np.argwhere(gpu_ids != ora_ids)
    for s, r in mism:
        io, ig = int(ora_ids[s, r]), int(gpu_ids[s, r])
        assert io >= 0, f"{label}: oracle has no allowed id at step {s} row {r} but GPU chose {ig}"
        p = p_row(int(s), int(r))
        assert 0 <= ig < p.shape[0] and np.isfinite(p[ig]), f"{label}: GPU id {ig} is not a candidate (s={s}, r={r})"
        gap = float(p[io]) - float(p[ig])
        assert gap < NEAR_TIE_REL * (1 + abs(float(p[io]))), \
            f"{label}: step {s} row {r}: GPU {ig} (p={p[ig]}) vs oracle {io} (p={p[io]}), gap {gap}"
    frac = 1.0 - len(mism) / gpu_ids.size
    assert frac >= ID_MATCH_MIN, f"{label}: only {frac:.5f} of rows identical"
    return len(mism)


def check_tiles(gmax, garg, omax, oarg, p_rows, bounds, label=""):
    """Per-tile maxima [R, n_tiles] vs the oracle's; p_rows[r] = oracle perturbed scores of row r."""
    gmax = np.asarray(gmax, np.float64)
    omax = np.asarray(omax, np.float64)
    fin = np.isfinite(omax)
    assert np.array_equal(fin, np.isfinite(gmax)), f"{label}: finite pattern differs"
    err = np.abs(gmax[fin] - omax[fin]) / np.maximum(1.0, np.abs(omax[fin]))
    assert err.size == 0 or err.max() <= TILE_REL, f"{label}: tile max rel err {err.max()}"
    for r, t in np.argwhere(np.asarray(garg) != np.asarray(oarg)):
        p = p_rows[r]
        io, ig = int(oarg[r, t]), int(garg[r, t])
        assert bounds[t] <= ig < bounds[t + 1], f"{label}: tile arg {ig} outside tile {t}"
        assert p[io] - p[ig] < NEAR_TIE_REL * (1 + abs(float(p[io]))), f"{label}: tile {t} row {r} arg mismatch"
    return float(err.max()) if err.size else 0.0


def kth_score(s_all, k):
    """k-th largest finite score of a row (-inf if fewer than k are finite)."""
    fin = np.sort(s_all[np.isfinite(s_all)].astype(np.float64))[::-1]
    return float(fin[k - 1]) if fin.size >= k else -np.inf


def nucleus_shares(s_all, top_k):
    """{id: share of the kept mass held by the ids ahead of it} over the top-k ids of a row
    (scores descending, lower id first), in fp64."""
    fin = np.flatnonzero(np.isfinite(s_all))
    order = fin[np.lexsort((fin, -s_all[fin]))][:top_k]
    if order.size == 0:
        return {}
    w = np.exp(s_all[order] - s_all[order[0]])
    before = np.concatenate([[0.0], np.cumsum(w)[:-1]]) / w.sum()
    return dict(zip(order.tolist(), before.tolist()))


def check_ids_topk(gpu_ids, ora_ids, L_rows, rows, T, seed, step0, top_k, mask=None, label="", top_p=1.0):
    """check_ids for top-k (and top-p) sampling, with the boundary readings of the near-tie rule.

    gpu_ids, ora_ids: [S, R]; L_rows[r] are the oracle's logits of global row rows[r].  A
    mismatch is accepted if it is a near tie of the final argmax among the oracle's kept ids,
    or if the kept sets may differ at the k-th boundary: the GPU's id or the oracle's has a
    score within 1e-3 (1 + |s_k|) of the k-th largest score s_k, or, with top_p < 1, at the
    nucleus boundary: the share of the kept mass ahead of the GPU's id or the oracle's is
    within 1e-3 of top_p.  The GPU's id must always be an allowed id whose score reaches s_k
    and whose share ahead stays below top_p, up to those tolerances.  Returns the count.
    """
    gpu_ids = np.asarray(gpu_ids)
    ora_ids = np.asarray(ora_ids)
    assert gpu_ids.shape == ora_ids.shape
    mism = np.argwhere(gpu_ids != ora_ids)
    for s, r in mism:
        io, ig = int(ora_ids[s, r]), int(gpu_ids[s, r])
        mrow = None if mask is None else mask[rows[r]]
        s_all = oracle.scores_row(L_rows[r], T, mask_row=mrow).astype(np.float64)
        assert io >= 0, f"{label}: oracle has no allowed id at step {s} row {r} but GPU chose {ig}"
        assert 0 <= ig < s_all.shape[0] and np.isfinite(s_all[ig]), f"{label}: GPU id {ig} not allowed"
        sk = kth_score(s_all, top_k)
        tol_k = NEAR_TIE_REL * (1 + abs(sk)) if np.isfinite(sk) else 0.0
        assert s_all[ig] >= sk - tol_k, f"{label}: GPU id {ig} (s={s_all[ig]}) below the k-th score {sk}"
        p = oracle.perturbed_row(L_rows[r], T, seed, step0 + int(s), int(rows[r]), mask_row=mrow, top_k=top_k,
                                 top_p=top_p)
        final_tie = np.isfinite(p[ig]) and float(p[io]) - float(p[ig]) < NEAR_TIE_REL * (1 + abs(float(p[io])))
        boundary = abs(s_all[ig] - sk) < tol_k or abs(s_all[io] - sk) < tol_k
        if top_p < 1.0:
            sh = nucleus_shares(s_all, top_k)
            last = max(sh.values())
            share_g, share_o = sh.get(ig, last), sh.get(io, last)
            assert share_g < top_p + NEAR_TIE_REL, f"{label}: GPU id {ig} outside the nucleus (share {share_g})"
            boundary = boundary or abs(share_g - top_p) < NEAR_TIE_REL or abs(share_o - top_p) < NEAR_TIE_REL
        assert final_tie or boundary, \
            f"{label}: step {s} row {r}: GPU {ig} vs oracle {io} (s {s_all[ig]} / {s_all[io]}, s_k {sk})"
    frac = 1.0 - len(mism) / gpu_ids.size
    assert frac >= ID_MATCH_MIN, f"{label}: only {frac:.5f} of rows identical"
    return len(mism)


def oracle_p_fn(L_rows, rows, T, seed, step0, mask=None, top_k=0):
    """p_row(s, r) for check_ids: oracle perturbed scores of L_rows[r] (global row rows[r]) at step0 + s."""
    def p_row(s, r):
        mrow = None if mask is None else mask[rows[r]]
        return oracle.perturbed_row(L_rows[r], T, seed, step0 + s, int(rows[r]), mask_row=mrow, top_k=top_k)

    return p_row
