"""GPU parity at the decode-head workloads' full sizes, in the benchmark's launch
configuration (default path and tiling), on sampled rows the oracle computes
one by one.

  small decode head  d=2048, V=151936, B in {1..64}, T=1.0, up to 1000 steps
  mid decode head    d=4096, V=151936, B in {1, 8, 32, 64, 128, 256}, T=0.7
  masked             d=5120, V=151936, B=32, 30% of ids disallowed, W outliers
  grouped            d=7168, V=262144 = 8 x 32768, B=64
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_ids, check_tiles, dev_bf16, dev_words, oracle_p_fn, say

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

    c = fs.fs_create(0, max_B=256, max_V=262144, max_top_k=64)
    torch.cuda.synchronize()
    yield c
    torch.cuda.synchronize()
    fs.fs_destroy(c)


def _sync():
    import torch

    torch.cuda.synchronize()


class Workload:
    def __init__(self, name):
        say(f"generating {name} weights")
        self.name = name
        self.w = synth.WORKLOADS[name]
        self.W = synth.workload_W(name)
        self.Wd = dev_bf16(self.W)
        say(f"{name}: W {self.W.shape} on device")


@pytest.fixture(scope="module")
def small(fs):
    return Workload("small_decode")


@pytest.fixture(scope="module")
def mid(fs):
    return Workload("mid_decode")


def _sample_rows(B):
    return np.unique(np.array([0, B // 2, B - 1], np.int32))


def _parity_run(fs, ctx, wl, B, T, steps, mask=None, seed=0, top_k=0):
    import torch

    H = synth.workload_H(wl.name, B=B)
    Hd = dev_bf16(H)
    md = None if mask is None else dev_words(mask)
    say(f"{wl.name} B={B} top_k={top_k}: {steps} GPU steps")
    outs = [fs.fs_fmms_sample(ctx, Hd, wl.Wd, T, seed, s, mask=md, top_k=top_k) for s in range(steps)]
    _sync()
    gpu = torch.stack(outs).cpu().numpy()
    rows = _sample_rows(B)
    say(f"{wl.name} B={B}: oracle logits for rows {rows.tolist()}")
    L = oracle.logits(H[rows], wl.W)
    ora, _ = oracle.sample_rows_steps(L, rows, T, seed, 0, steps, mask=mask, top_k=top_k)
    n = check_ids(gpu[:, rows], ora, oracle_p_fn(L, rows, T, seed, 0, mask=mask, top_k=top_k),
                  f"{wl.name} B={B} top_k={top_k}")
    say(f"{wl.name} B={B}: {steps}x{len(rows)} sampled rows, near-tie mismatches {n}")
    return gpu, H, L, rows


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_small_decode_head(fs, ctx, small, B):
    _parity_run(fs, ctx, small, B, 1.0, 1000 if B == 64 else 100)


@pytest.mark.parametrize("B", [1, 8, 32, 64, 128, 256])
def test_mid_decode_head(fs, ctx, mid, B):
    _parity_run(fs, ctx, mid, B, 0.7, 100)


@pytest.mark.parametrize("B", [8, 64])
def test_mid_decode_head_topk50(fs, ctx, mid, B):
    # the mid decode head's top-k variant: exact top-50 of the scores, then the
    # Gumbel-max within them
    gpu, _, L, rows = _parity_run(fs, ctx, mid, B, 0.7, 20, top_k=50)
    for j, r in enumerate(rows):  # every draw lies in the oracle's top-50 set
        kept = set(np.argsort(-L[j].astype(np.float64), kind="stable")[:50].tolist())
        assert set(gpu[:, r].tolist()) <= kept


def test_mid_decode_tile_maxima(fs, ctx, mid):
    import torch

    B = 64
    H = synth.workload_H("mid_decode", B=B)
    nt, bounds = fs.fs_fmms_tiling(ctx, B, H.shape[1], mid.W.shape[0])
    say(f"mid decode tile maxima B={B} n_tiles={nt}")
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    fs.fs_fmms_sample(ctx, dev_bf16(H), mid.Wd, 0.7, 0, 3, tile_max=tmax, tile_arg=targ)
    _sync()
    rows = _sample_rows(B)
    L = oracle.logits(H[rows], mid.W)
    bnd = np.array(bounds, np.int64)
    p_rows = [oracle.perturbed_row(L[i], 0.7, 0, 3, int(r)) for i, r in enumerate(rows)]
    omax = np.empty((len(rows), nt), np.float32)
    oarg = np.empty((len(rows), nt), np.int32)
    for i, p in enumerate(p_rows):
        for t in range(nt):
            a = int(np.argmax(p[bnd[t]:bnd[t + 1]]))
            omax[i, t] = p[bnd[t] + a]
            oarg[i, t] = bnd[t] + a
    err = check_tiles(tmax.cpu().numpy()[rows], targ.cpu().numpy()[rows], omax, oarg, p_rows, bnd, "mid tiles")
    say(f"max tile rel err {err:.2e}")


def test_masked_workload(fs, ctx):
    wl = Workload("masked")
    B = wl.w["B"]
    mask = synth.workload_mask("masked")
    allowed = synth.unpack_mask(mask, wl.W.shape[0])
    gpu, _, _, _ = _parity_run(fs, ctx, wl, B, 1.0, 100, mask=mask)
    for b in range(B):
        assert np.all(allowed[b, gpu[:, b]]), f"masked id drawn in row {b}"


def test_grouped_workload(fs, ctx):
    import torch

    wl = Workload("grouped")
    B, n_groups, T = wl.w["B"], wl.w["n_groups"], 1.0
    V = wl.W.shape[0]
    G = V // n_groups
    H = synth.workload_H("grouped")
    Hd = dev_bf16(H)
    rows = _sample_rows(B)
    say(f"grouped: oracle logits for rows {rows.tolist()}")
    L = oracle.logits(H[rows], wl.W)
    steps = 12
    for step in range(steps):
        summ = torch.empty((n_groups, B, 3), dtype=torch.int32, device="cuda")
        for k in range(n_groups):
            fs.fs_group_summary(ctx, Hd, wl.Wd[k * G:(k + 1) * G], k * G, T, 0, step, out=summ[k])
        flat = fs.fs_fmms_sample(ctx, Hd, wl.Wd, T, 0, step)
        comb_m = fs.fs_group_combine(ctx, summ, 0, step, fs.FS_COMBINE_MAX)
        comb_g = fs.fs_group_combine(ctx, summ, 0, step, fs.FS_COMBINE_GUMBEL)
        _sync()
        assert torch.equal(comb_m, flat)
        lse, pmax, arg = (x.cpu().numpy() for x in fs.summary_views(summ))
        # flat sample on sampled rows vs the oracle
        ora, _ = oracle.sample_rows_steps(L, rows, T, 0, step, 1)
        check_ids(flat.cpu().numpy()[rows][None, :], ora, oracle_p_fn(L, rows, T, 0, step), "grouped flat")
        for i, r in enumerate(rows):
            p = oracle.perturbed_row(L[i], T, 0, step, int(r))
            s = (L[i] / np.float32(T)).astype(np.float64)
            for k in range(n_groups):
                seg = slice(k * G, (k + 1) * G)
                m = s[seg].max()
                olse = m + np.log(np.exp(s[seg] - m).sum())
                assert abs(lse[k, r] - olse) <= 1e-4 * max(1.0, abs(olse))
                assert abs(pmax[k, r] - p[seg].max()) <= 1e-3 * max(1.0, abs(p[seg].max()))
                oa = k * G + int(np.argmax(p[seg]))
                if arg[k, r] != oa:
                    assert p[oa] - p[arg[k, r]] < 1e-3 * (1 + abs(p[oa]))
        ref_g = oracle.group_combine(lse, pmax, arg, 0, step, oracle.GROUP_MODE_GUMBEL)
        assert np.mean(ref_g == comb_g.cpu().numpy()) >= 0.999 or np.sum(ref_g != comb_g.cpu().numpy()) <= 1
    say(f"grouped: {steps} steps ok")


def test_mid_decode_head_masked_b64(fs, ctx, mid):
    # four batch blocks with a mask: the chunk-outer kernel's masked form, two passes per tile
    B = 64
    mask = synth.bernoulli_mask(B, mid.W.shape[0], 901, 0.3)
    allowed = synth.unpack_mask(mask, mid.W.shape[0])
    gpu, _, _, _ = _parity_run(fs, ctx, mid, B, 0.7, 20, mask=mask)
    for b in range(B):
        assert np.all(allowed[b, gpu[:, b]]), f"masked id drawn in row {b}"


def test_mid_decode_group_summary_b64(fs, ctx, mid):
    # one large group (131072 ids: several rounds per tile) at four batch blocks
    import torch

    B, G, T = 64, 131072, 0.7
    H = synth.workload_H("mid_decode", B=B)
    Hd = dev_bf16(H)
    rows = _sample_rows(B)
    L = oracle.logits(H[rows], mid.W[:G])
    summ = torch.empty((B, 3), dtype=torch.int32, device="cuda")
    for step in (0, 1):
        fs.fs_group_summary(ctx, Hd, mid.Wd[:G], 0, T, 0, step, out=summ)
        _sync()
        lse, pmax, arg = (x.cpu().numpy() for x in fs.summary_views(summ))
        for i, r in enumerate(rows):
            p = oracle.perturbed_row(L[i], T, 0, step, int(r))
            s = (L[i] / np.float32(T)).astype(np.float64)
            m = s.max()
            olse = m + np.log(np.exp(s - m).sum())
            assert abs(lse[r] - olse) <= 1e-4 * max(1.0, abs(olse))
            assert abs(pmax[r] - p.max()) <= 1e-3 * max(1.0, abs(p.max()))
            oa = int(np.argmax(p))
            if arg[r] != oa:
                assert p[oa] - p[arg[r]] < 1e-3 * (1 + abs(p[oa]))
    say(f"group summary B={B} G={G}: ok")
