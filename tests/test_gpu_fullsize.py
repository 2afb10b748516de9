"""GPU parity at the decode-head workloads' full sizes, in the benchmark's launch
configuration (default path and tiling), on every batch row.

  small decode head  d=2048, V=151936, B in {1..64}, T=1.0, 1000 steps each
  mid decode head    d=4096, V=151936, B in {1, 8, 32, 64, 128, 256}, T=0.7,
                     plus the top-50 variant at B in {1, 8, 32, 64, 128}
  masked             d=5120, V=151936, B=32, 30% of ids disallowed, W outliers
  grouped            d=7168, V=262144 = 8 x 32768, B=64

The oracle's logits do not depend on the step, so they are computed once per
workload for the largest batch (the hidden states of a smaller batch are the
first rows of a larger one) and only the noise and argmax run per step.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (NEAR_TIE_REL, check_ids, check_ids_topk, check_tiles, dev_bf16, dev_words, oracle_p_fn,
                         say)

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
    """Weights on the device and the oracle's logits of the first `rows` hidden-state rows."""

    def __init__(self, name, rows):
        say(f"generating {name} weights")
        self.name = name
        self.w = synth.WORKLOADS[name]
        self.W = synth.workload_W(name)
        self.Wd = dev_bf16(self.W)
        self.H = synth.workload_H(name, B=rows)
        say(f"{name}: W {self.W.shape} on device; oracle logits of {rows} rows")
        self.L = oracle.logits(self.H, self.W)
        say(f"{name}: oracle logits ready")


@pytest.fixture(scope="module")
def small(fs):
    return Workload("small_decode", 64)


@pytest.fixture(scope="module")
def mid(fs):
    return Workload("mid_decode", 256)


def _parity_run(fs, ctx, wl, B, T, steps, mask=None, seed=0, top_k=0):
    import torch

    H = wl.H[:B]
    assert np.array_equal(H, synth.workload_H(wl.name, B=B))
    Hd = dev_bf16(H)
    md = None if mask is None else dev_words(mask)
    say(f"{wl.name} B={B} top_k={top_k}: {steps} GPU steps")
    outs = [fs.fs_fmms_sample(ctx, Hd, wl.Wd, T, seed, s, mask=md, top_k=top_k) for s in range(steps)]
    _sync()
    gpu = torch.stack(outs).cpu().numpy()
    rows = np.arange(B, dtype=np.int32)
    L = wl.L[:B]
    say(f"{wl.name} B={B}: oracle samples of all {B} rows x {steps} steps")
    ora, _ = oracle.sample_rows_steps(L, rows, T, seed, 0, steps, mask=mask, top_k=top_k)
    label = f"{wl.name} B={B} top_k={top_k}"
    if top_k:
        n = check_ids_topk(gpu, ora, L, rows, T, seed, 0, top_k, mask=mask, label=label)
    else:
        n = check_ids(gpu, ora, oracle_p_fn(L, rows, T, seed, 0, mask=mask), label)
    say(f"{label}: {steps}x{B} rows, near-tie mismatches {n}")
    return gpu, H, L, rows


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_small_decode_head(fs, ctx, small, B):
    # 1000 consecutive steps, step counter incrementing, every row
    _parity_run(fs, ctx, small, B, 1.0, 1000)


@pytest.mark.parametrize("B", [1, 8, 32, 64, 128, 256])
def test_mid_decode_head(fs, ctx, mid, B):
    # every row: at B=128 and 256 every lane position of every 16-row batch
    # block of the 128-column kernel is compared
    _parity_run(fs, ctx, mid, B, 0.7, 100 if B <= 64 else 40)


@pytest.mark.parametrize("B", [1, 8, 32, 64, 128])
def test_mid_decode_head_topk50(fs, ctx, mid, B):
    # the mid decode head's top-k variant: exact top-50 of the scores, then the
    # Gumbel-max within them, against the oracle's own logits
    gpu, _, L, rows = _parity_run(fs, ctx, mid, B, 0.7, 20, top_k=50)
    for j, r in enumerate(rows):  # every draw reaches the oracle's 50th score up to the tolerance
        s = L[j].astype(np.float64) / 0.7
        sk = np.sort(s)[::-1][49]
        assert np.all(s[gpu[:, r]] >= sk - NEAR_TIE_REL * (1 + abs(sk)))


def test_mid_decode_tile_maxima(fs, ctx, mid):
    import torch

    B = 64
    H = mid.H[:B]
    nt, bounds = fs.fs_fmms_tiling(ctx, B, H.shape[1], mid.W.shape[0])
    say(f"mid decode tile maxima B={B} n_tiles={nt}")
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    fs.fs_fmms_sample(ctx, dev_bf16(H), mid.Wd, 0.7, 0, 3, tile_max=tmax, tile_arg=targ)
    _sync()
    rows = np.arange(B)
    L = mid.L[:B]
    bnd = np.array(bounds, np.int64)
    omax, oarg = oracle.tile_maxima(L, 0.7, 0, 3, bnd)
    p_rows = [oracle.perturbed_row(L[i], 0.7, 0, 3, int(r)) for i, r in enumerate(rows)]
    err = check_tiles(tmax.cpu().numpy(), targ.cpu().numpy(), omax, oarg, p_rows, bnd, "mid tiles")
    say(f"max tile rel err {err:.2e}")


def test_masked_workload(fs, ctx):
    wl = Workload("masked", synth.WORKLOADS["masked"]["B"])
    B = wl.w["B"]
    mask = synth.workload_mask("masked")
    allowed = synth.unpack_mask(mask, wl.W.shape[0])
    gpu, _, _, _ = _parity_run(fs, ctx, wl, B, 1.0, 100, mask=mask)
    for b in range(B):
        assert np.all(allowed[b, gpu[:, b]]), f"masked id drawn in row {b}"


def _group_noise(seed, step, b, n_groups):
    return np.array([oracle.gumbel32(oracle.group_noise_bits(seed, step, int(b), k)) for k in range(n_groups)])


def test_grouped_workload(fs, ctx):
    import torch

    wl = Workload("grouped", synth.WORKLOADS["grouped"]["B"])
    B, n_groups, T = wl.w["B"], wl.w["n_groups"], 1.0
    V = wl.W.shape[0]
    G = V // n_groups
    Hd = dev_bf16(wl.H)
    rows = np.arange(B)
    L = wl.L
    steps = 12
    comb_mism = comb_draws = 0
    flats = []
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
        flats.append(flat.cpu().numpy())
        for k in range(n_groups):
            olse, opmax, oarg = oracle.group_summary(L, k * G, G, T, 0, step)
            assert np.all(np.abs(lse[k] - olse) <= 1e-4 * np.maximum(1.0, np.abs(olse)))
            assert np.all(np.abs(pmax[k] - opmax) <= 1e-3 * np.maximum(1.0, np.abs(opmax)))
            for b in np.flatnonzero(arg[k] != oarg):
                p = oracle.perturbed_row(L[b], T, 0, step, int(b))
                assert p[oarg[b]] - p[arg[k, b]] < NEAR_TIE_REL * (1 + abs(float(p[oarg[b]])))
        # the oracle's Gumbel combine on the GPU's summaries, at this step and at 63 more
        # combine steps over the same summaries (the combine's noise is all that changes):
        # a differing row must be a near tie of the group keys lse_k + g'_k
        for cstep in [step] + list(range(1000 + 64 * step, 1000 + 64 * step + 63)):
            got_g = (comb_g if cstep == step else fs.fs_group_combine(ctx, summ, 0, cstep, fs.FS_COMBINE_GUMBEL))
            got_g = got_g.cpu().numpy()
            ref_g = oracle.group_combine(lse, pmax, arg, 0, cstep, oracle.GROUP_MODE_GUMBEL)
            for b in np.flatnonzero(ref_g != got_g):
                keys = lse[:, b].astype(np.float64) + _group_noise(0, cstep, b, n_groups)
                srt = np.sort(keys)[::-1]
                assert srt[0] - srt[1] < NEAR_TIE_REL * (1 + abs(srt[0])), f"grouped combine row {b} step {cstep}"
                comb_mism += 1
            comb_draws += B
    assert comb_mism <= 0.001 * comb_draws, f"grouped combine: {comb_mism} of {comb_draws} draws differ"
    # the flat sample of every row and step vs the oracle
    ora, _ = oracle.sample_rows_steps(L, rows, T, 0, 0, steps)
    check_ids(np.stack(flats), ora, oracle_p_fn(L, rows, T, 0, 0), "grouped flat")
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
    Hd = dev_bf16(mid.H[:B])
    L = np.ascontiguousarray(mid.L[:B, :G])
    summ = torch.empty((B, 3), dtype=torch.int32, device="cuda")
    for step in (0, 1):
        fs.fs_group_summary(ctx, Hd, mid.Wd[:G], 0, T, 0, step, out=summ)
        _sync()
        lse, pmax, arg = (x.cpu().numpy() for x in fs.summary_views(summ))
        olse, opmax, oarg = oracle.group_summary(L, 0, G, T, 0, step)
        assert np.all(np.abs(lse - olse) <= 1e-4 * np.maximum(1.0, np.abs(olse)))
        assert np.all(np.abs(pmax - opmax) <= 1e-3 * np.maximum(1.0, np.abs(opmax)))
        for b in np.flatnonzero(arg != oarg):
            p = oracle.perturbed_row(L[b], T, 0, step, int(b))
            assert p[oarg[b]] - p[arg[b]] < NEAR_TIE_REL * (1 + abs(float(p[oarg[b]])))
    say(f"group summary B={B} G={G}: ok")
