"""GPU parity of the HIP library against the CPU oracle (small and ragged shapes).

Every test calls the library through its C ABI (via the ctypes binding) and
compares with the oracle on the same seeded inputs from `synth`:
  * Philox words bit for bit, Gumbel values to ~1e-6, the transform finite on
    all 2^32 words (device scan);
  * logits bit for bit on integer-valued inputs (checks the MFMA operand and
    accumulator layouts);
  * sampled ids: identical on >= 99.9% of rows, every mismatch a near-tie
    (oracle perturbed scores within 1e-3 (1 + |max|));
  * per-tile maxima within 1e-3 relative;
  * unfused path == fused path bit for bit; grouped summaries, both combines.
"""
import math

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

    c = fs.fs_create(0, max_B=320, max_V=262144, max_top_k=64)
    torch.cuda.synchronize()
    yield c
    torch.cuda.synchronize()
    fs.fs_destroy(c)


def _sync():
    import torch

    torch.cuda.synchronize()


# --- noise ---------------------------------------------------------------------

@pytest.mark.parametrize("seed,step,row,v0,n", [
    (0, 0, 0, 0, 4096),
    (123456789012345, 7, 3, 1000, 777),
    (2**64 - 1, 2**40 + 5, 255, 2**31 - 4096, 4096),
])
def test_philox_words_bitwise(fs, ctx, seed, step, row, v0, n):
    say(f"philox seed={seed} step={step} row={row} v0={v0} n={n}")
    r, g = fs.fs_debug_philox(ctx, seed, step, row, v0, n)
    _sync()
    got = r.cpu().numpy().view(np.uint32)
    ref = oracle.noise_bits_range(seed, step, row, v0, n)
    assert np.array_equal(got, ref)
    gref = np.array([oracle.gumbel32(int(x)) for x in ref], np.float32)
    assert np.max(np.abs(g.cpu().numpy() - gref)) < 2e-6 * 23


def test_gumbel_values_match_oracle(fs, ctx):
    # words at both ends (u -> 0 and u -> 1), around the branch at 2^31 and the
    # series/log switch, and a stride across the rest
    spans = [(0, 1 << 20), ((1 << 31) - (1 << 19), 1 << 20), ((1 << 32) - (1 << 20), 1 << 20),
             ((1 << 32) - (1 << 28) - (1 << 16), 1 << 17)]
    worst = 0.0
    for r0, n in spans:
        say(f"gumbel span r0={r0} n={n}")
        g = fs.fs_debug_gumbel_bits(ctx, r0, n)
        _sync()
        ref = oracle.gumbel32_range(r0, n).astype(np.float64)
        err = np.abs(g.cpu().numpy().astype(np.float64) - ref)
        worst = max(worst, float(err.max()))
    for r0 in range(0, 1 << 32, 1 << 26):  # 64 short runs spread over all words
        g = fs.fs_debug_gumbel_bits(ctx, r0, 4096)
        _sync()
        ref = oracle.gumbel32_range(r0, 4096).astype(np.float64)
        worst = max(worst, float(np.abs(g.cpu().numpy().astype(np.float64) - ref).max()))
    say(f"max |g_gpu - g_oracle| = {worst:.3e}")
    assert worst < 1e-5


def test_gumbel_exhaustive_scan_finite(fs, ctx):
    say("gumbel exhaustive scan over 2^32 words")
    st = fs.fs_debug_gumbel_scan(ctx)
    _sync()
    st = st.cpu().numpy().astype(np.uint64)
    nonfinite, decreases = int(st[0]), int(st[1])
    gmin = float(np.array([st[2]], np.uint64).astype(np.uint32).view(np.float32)[0])
    gmax = float(np.array([st[3]], np.uint64).astype(np.uint32).view(np.float32)[0])
    say(f"nonfinite={nonfinite} decreases={decreases} min={gmin} max={gmax}")
    assert nonfinite == 0
    assert abs(gmin - (-math.log(math.log(2.0**32 + 1)))) < 1e-5
    assert abs(gmax - (-math.log(math.log1p(2.0**-32)))) < 1e-4
    # the device transform is monotone in the word: no word's noise is below its predecessor's
    assert decreases == 0


# --- exact logits --------------------------------------------------------------

@pytest.mark.parametrize("B,d,V,path", [
    (2, 256, 1000, 1), (5, 256, 1000, 2), (20, 264, 777, 2), (64, 512, 1030, 2), (1, 1000, 333, 1),
    (3, 2056, 515, 0), (64, 2056, 300, 2),
])
def test_logits_exact_on_integer_inputs(fs, ctx, B, d, V, path):
    import torch

    say(f"exact logits B={B} d={d} V={V} path={path}")
    H = synth.small_int_bf16(B, d, seed=1)
    W = synth.small_int_bf16(V, d, seed=2, lo=-1, hi=1)
    Lref = oracle.logits(H, W)
    assert np.abs(Lref).max() < 2**24  # every partial sum is exact in fp32
    ws = torch.full((B, (V + 3) // 4 * 4), float("nan"), dtype=torch.float32, device="cuda")
    fs.fs_unfused_sample(ctx, dev_bf16(H), dev_bf16(W), 1.0, 0, 0, logits_ws=ws, path=path)
    _sync()
    got = ws.cpu().numpy()[:, :V]
    assert np.array_equal(got, Lref)


# --- sampling parity -------------------------------------------------------------

def _run_steps(fs, ctx, Hd, Wd, T, seed, steps, mask=None, path=0):
    import torch

    outs = []
    for s in steps:
        outs.append(fs.fs_fmms_sample(ctx, Hd, Wd, T, seed, s, mask=mask, path=path))
    _sync()
    return torch.stack(outs).cpu().numpy()


@pytest.mark.parametrize("path", [0, 1, 2])
def test_tiny_workload_parity(fs, ctx, path):
    w = synth.WORKLOADS["tiny"]
    say(f"tiny workload B={w['B']} d={w['d']} V={w['V']} path={path}, 200 steps")
    H = synth.workload_H("tiny")
    if path == 1:  # the dot-product kernel takes at most 2 rows
        H = H[:2]
    W = synth.workload_W("tiny")
    L = oracle.logits(H, W)
    gpu = _run_steps(fs, ctx, dev_bf16(H), dev_bf16(W), 1.0, 0, range(200), path=path)
    rows = np.arange(H.shape[0])
    ora, _ = oracle.sample_rows_steps(L, rows, 1.0, 0, 0, 200)
    n = check_ids(gpu, ora, oracle_p_fn(L, rows, 1.0, 0, 0), "tiny")
    say(f"near-tie mismatches: {n}")


@pytest.mark.parametrize("path", [1, 2])
def test_tile_maxima_tiny(fs, ctx, path):
    import torch

    H = synth.workload_H("tiny")
    if path == 1:
        H = H[:2]
    W = synth.workload_W("tiny")
    L = oracle.logits(H, W)
    B, V = L.shape
    nt, bounds = fs.fs_fmms_tiling(ctx, B, H.shape[1], V, path)
    say(f"tile maxima tiny path={path} n_tiles={nt}")
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    for step in (0, 1, 17):
        fs.fs_fmms_sample(ctx, dev_bf16(H), dev_bf16(W), 1.0, 0, step, tile_max=tmax, tile_arg=targ, path=path)
        _sync()
        omax, oarg = oracle.tile_maxima(L, 1.0, 0, step, np.array(bounds))
        p_rows = [oracle.perturbed_row(L[b], 1.0, 0, step, b) for b in range(B)]
        check_tiles(tmax.cpu().numpy(), targ.cpu().numpy(), omax, oarg, p_rows, bounds, f"tiles step {step}")


RAGGED = [
    # B, d, V, T, path
    (1, 264, 1000, 1.0, 0), (1, 264, 1000, 1.0, 2), (3, 1000, 4097, 0.7, 0), (3, 1000, 4097, 0.7, 2),
    (2, 512, 333, 1.3, 1), (7, 512, 333, 1.3, 0), (8, 512, 2000, 1.0, 0), (17, 256, 2000, 0.9, 0), (33, 520, 1234, 1.0, 0),
    (48, 768, 3001, 0.7, 0), (64, 2056, 1500, 1.0, 0), (65, 256, 999, 1.0, 0), (100, 264, 777, 0.8, 0),
    (2, 86016, 300, 1.0, 1), (2, 16, 7, 1.0, 0), (16, 20480, 300, 1.0, 2),
    # rows of more than 8 sub-blocks with H resident: the kernel with the tile's noise table
    (5, 3072, 3001, 0.8, 0), (16, 2560, 2049, 1.0, 0), (1, 4096, 5000, 1.0, 0),
    # the wide kernel (65 .. 256 rows, d a multiple of 256): eight batch blocks
    # and sixteen, rows past B in the last block, tiles of one vocab block (the
    # other waves' slots empty), a batch split into 256 rows and a tail of 44
    # or 1, and tiles of three and four passes (up to 20 blocks a pass: ~49
    # and 64 blocks a tile) with a ragged last vocab block
    (65, 512, 999, 1.0, 0), (100, 1024, 777, 0.8, 0), (128, 2048, 4099, 0.7, 0), (129, 512, 1500, 1.0, 0),
    (200, 512, 3001, 0.9, 0), (256, 1024, 9001, 0.8, 0), (136, 512, 70001, 1.0, 0), (300, 512, 2000, 1.0, 0),
    (257, 512, 1000, 1.1, 0), (136, 256, 200003, 1.0, 0), (256, 256, 262143, 0.9, 0), (100, 256, 262143, 1.0, 0),
    # more than 64 rows with d not a multiple of 256: 64-row chunks
    (129, 264, 1500, 1.0, 0), (70, 520, 999, 1.0, 0),
    # more than 16 rows at d <= 2048: H in chunks although it would fit in LDS
    (24, 2048, 3001, 0.9, 0), (32, 1024, 2000, 1.0, 0),
]


@pytest.mark.parametrize("B,d,V,T,path", RAGGED)
def test_ragged_shapes_parity(fs, ctx, B, d, V, T, path):
    say(f"ragged B={B} d={d} V={V} T={T} path={path}")
    H = synth.normal_bf16(B, d, seed=100 + B)
    W = synth.normal_bf16(V, d, seed=200 + V, std=2.0 / math.sqrt(d))
    L = oracle.logits(H, W)
    steps = 12
    gpu = _run_steps(fs, ctx, dev_bf16(H), dev_bf16(W), T, 42, range(steps), path=path)
    rows = np.arange(B)
    ora, _ = oracle.sample_rows_steps(L, rows, T, 42, 0, steps)
    check_ids(gpu, ora, oracle_p_fn(L, rows, T, 42, 0), f"ragged {B}x{d}x{V}")


# Chunk-outer shapes with at least 16 blocks of 16 vocab rows per tile: calls
# without tile maxima run with XCD-weighted tiles, calls with them on the equal
# tiling; both samples are checked against the oracle.
XCD_TILED = [
    # B, d, V, T
    (24, 4096, 65551, 0.8), (40, 2048, 70001, 1.0), (40, 3072, 66000, 0.7),
    (16, 4096, 90007, 1.0),  # H would fit in LDS, its noise table beside it not: chunked H
]


@pytest.mark.parametrize("B,d,V,T", XCD_TILED)
def test_xcd_weighted_tiles_parity(fs, ctx, B, d, V, T):
    import torch

    say(f"XCD-weighted tiles B={B} d={d} V={V} T={T}")
    H = synth.normal_bf16(B, d, seed=300 + B)
    W = synth.normal_bf16(V, d, seed=400 + B, std=2.0 / math.sqrt(d))
    L = oracle.logits(H, W)
    steps = 6
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    gpu = _run_steps(fs, ctx, Hd, Wd, T, 9, range(steps))
    rows = np.arange(B)
    ora, _ = oracle.sample_rows_steps(L, rows, T, 9, 0, steps)
    check_ids(gpu, ora, oracle_p_fn(L, rows, T, 9, 0), f"weighted tiles {B}x{d}x{V}")
    nt, _ = fs.fs_fmms_tiling(ctx, B, d, V)
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    eq = torch.stack([fs.fs_fmms_sample(ctx, Hd, Wd, T, 9, s, tile_max=tmax, tile_arg=targ) for s in range(steps)])
    _sync()
    check_ids(eq.cpu().numpy(), ora, oracle_p_fn(L, rows, T, 9, 0), f"equal tiles {B}x{d}x{V}")


def test_strided_operands(fs, ctx):
    # ldh, ldw > d: row strides are honoured
    import torch

    B, d, V = 6, 256, 900
    say("strided operands")
    H = synth.normal_bf16(B, d, seed=5)
    W = synth.normal_bf16(V, d, seed=6, std=0.1)
    Hp = torch.zeros((B, d + 24), dtype=torch.bfloat16, device="cuda")
    Wp = torch.zeros((V, d + 40), dtype=torch.bfloat16, device="cuda")
    Hp[:, :d] = dev_bf16(H)
    Wp[:, :d] = dev_bf16(W)
    Hp[:, d:] = 1e4
    Wp[:, d:] = 1e4
    a = fs.fs_fmms_sample(ctx, Hp[:, :d], Wp[:, :d], 1.0, 3, 9)
    b = fs.fs_fmms_sample(ctx, dev_bf16(H), dev_bf16(W), 1.0, 3, 9)
    _sync()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,d,V", [
    (12, 520, 3000),
    (6, 4096, 3001),  # rows of more than 8 sub-blocks with a mask: H in chunks, one batch block
])
def test_masked_parity_and_no_masked_picks(fs, ctx, B, d, V):
    T = 1.0
    say(f"masked B={B} d={d} V={V}")
    H = synth.normal_bf16(B, d, seed=7)
    W = synth.outlier_bf16(V, d, 8, 9, 0.05, 0.5, 0.01)
    allowed = np.random.default_rng(10).random((B, V)) >= 0.3
    allowed[3] = False  # no allowed id: must sample -1
    allowed[4] = False
    allowed[4, V - 1] = True  # exactly one allowed id, in the ragged tail
    mask = synth.pack_mask(allowed)
    L = oracle.logits(H, W)
    for path in (0, 1, 2) if B <= 2 else (0, 2):
        gpu = _run_steps(fs, ctx, dev_bf16(H), dev_bf16(W), T, 5, range(30), mask=dev_words(mask), path=path)
        assert np.all(gpu[:, 3] == -1)
        assert np.all(gpu[:, 4] == V - 1)
        ok_rows = [b for b in range(B) if b != 3]
        for b in ok_rows:
            assert np.all(allowed[b, gpu[:, b]]), f"masked id drawn in row {b}"
        rows = np.arange(B)
        ora, _ = oracle.sample_rows_steps(L, rows, T, 5, 0, 30, mask=mask)
        check_ids(gpu, ora, oracle_p_fn(L, rows, T, 5, 0, mask=mask), "masked")


@pytest.mark.parametrize("B,d,V,path", [(2, 256, 4096, 1), (4, 256, 4096, 2), (40, 1024, 5000, 0),
                                        (64, 2048, 3000, 2), (130, 264, 700, 0),
                                        (24, 4096, 65551, 0)])  # XCD-weighted tiles without the mask
def test_unfused_equals_fused(fs, ctx, B, d, V, path):
    # The unfused path stores the logits and samples them in a second kernel.  Its
    # logits pass may run another kernel form than the fused call (another fp32
    # summation order: chunk rotation, lane k layout), so the ids agree with the
    # fused ones except at near ties of the oracle's perturbed scores.
    import torch

    say(f"unfused vs fused B={B} d={d} V={V} path={path}")
    Hh = synth.normal_bf16(B, d, seed=11)
    Wh = synth.normal_bf16(V, d, seed=12, std=0.05)
    H, W = dev_bf16(Hh), dev_bf16(Wh)
    allowed = np.random.default_rng(13).random((B, V)) >= 0.2
    mask_np = synth.pack_mask(allowed)
    m = dev_words(mask_np)
    L = None
    for mask, mnp in ((None, None), (m, mask_np)):
        fused = torch.stack([fs.fs_fmms_sample(ctx, H, W, 0.8, 1, step, mask=mask, path=path) for step in range(5)])
        unf = torch.stack([fs.fs_unfused_sample(ctx, H, W, 0.8, 1, step, mask=mask, path=path) for step in range(5)])
        _sync()
        a, b = fused.cpu().numpy(), unf.cpu().numpy()
        if not np.array_equal(a, b):
            L = oracle.logits(Hh, Wh) if L is None else L
            check_ids(b, a, oracle_p_fn(L, np.arange(B), 0.8, 1, 0, mask=mnp), "unfused vs fused")


def test_nan_weights_never_win(fs, ctx):
    # W rows poisoned with NaN give NaN logits: NaN fails every comparison, so
    # such ids are never sampled, and a row whose every score is NaN samples -1
    import torch

    B, d, V = 20, 512, 3001
    say(f"NaN-poisoned W B={B} d={d} V={V}")
    H = synth.normal_bf16(B, d, seed=50)
    W = synth.normal_bf16(V, d, seed=51, std=0.1)
    bad = np.random.default_rng(52).random(V) < 0.05
    bad[:5] = True  # the lowest ids too: a NaN never wins on the tie rule
    W[bad, 7] = 0x7FC0  # one NaN element per poisoned row
    L = oracle.logits(H, W)
    assert np.all(np.isnan(L[:, bad])) and not np.any(np.isnan(L[:, ~bad]))
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    for path in (0, 2):
        gpu = _run_steps(fs, ctx, Hd, Wd, 1.0, 6, range(10), path=path)
        assert not np.any(bad[gpu]), "a NaN-scored id was sampled"
        rows = np.arange(B)
        ora, _ = oracle.sample_rows_steps(L, rows, 1.0, 6, 0, 10)
        check_ids(gpu, ora, oracle_p_fn(L, rows, 1.0, 6, 0), "NaN weights")
    # every score NaN (a NaN in each hidden-state row): no id can win
    Hn = H.copy()
    Hn[:, 3] = 0x7FC0
    out = fs.fs_fmms_sample(ctx, dev_bf16(Hn), Wd, 1.0, 6, 0)
    _sync()
    assert torch.all(out == -1)


def test_determinism_reruns(fs, ctx):
    import torch

    B, d, V = 64, 2048, 20000
    say(f"determinism B={B} d={d} V={V} x50")
    H = dev_bf16(synth.normal_bf16(B, d, seed=14))
    W = dev_bf16(synth.normal_bf16(V, d, seed=15, std=0.02))
    nt, _ = fs.fs_fmms_tiling(ctx, B, d, V)
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    ref = fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, tile_max=tmax, tile_arg=targ).clone()
    ref_t = tmax.clone()
    for _ in range(50):
        out = fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, tile_max=tmax, tile_arg=targ)
        assert torch.equal(out, ref) and torch.equal(tmax, ref_t)
    _sync()


# --- grouped ---------------------------------------------------------------------

@pytest.mark.parametrize("B,d,G,n_groups,path", [(6, 256, 512, 8, 0), (64, 768, 1024, 4, 0), (2, 512, 96, 5, 1)])
def test_grouped_summaries_and_combine(fs, ctx, B, d, G, n_groups, path):
    import torch

    V = G * n_groups
    say(f"grouped B={B} d={d} G={G} groups={n_groups} path={path}")
    H = synth.normal_bf16(B, d, seed=16)
    W = synth.normal_bf16(V, d, seed=17, std=1.5 / math.sqrt(d))
    allowed = np.random.default_rng(18).random((B, V)) >= 0.25
    mask = synth.pack_mask(allowed)
    L = oracle.logits(H, W)
    Hd, Wd, md = dev_bf16(H), dev_bf16(W), dev_words(mask)
    T, seed = 0.9, 77
    for step in range(4):
        summ = torch.empty((n_groups, B, 3), dtype=torch.int32, device="cuda")
        for k in range(n_groups):
            fs.fs_group_summary(ctx, Hd, Wd[k * G:(k + 1) * G], k * G, T, seed, step, mask=md, out=summ[k],
                                path=path)
        flat = fs.fs_fmms_sample(ctx, Hd, Wd, T, seed, step, mask=md, path=path)
        comb_m = fs.fs_group_combine(ctx, summ, seed, step, fs.FS_COMBINE_MAX)
        comb_g = fs.fs_group_combine(ctx, summ, seed, step, fs.FS_COMBINE_GUMBEL)
        _sync()
        assert torch.equal(comb_m, flat), "max-combine must equal the flat sample"
        lse, pmax, arg = (x.cpu().numpy() for x in fs.summary_views(summ))
        olse = np.empty((n_groups, B), np.float32)
        opmax = np.empty((n_groups, B), np.float32)
        oarg = np.empty((n_groups, B), np.int32)
        for k in range(n_groups):
            olse[k], opmax[k], oarg[k] = oracle.group_summary(L, k * G, G, T, seed, step, mask=mask)
        assert np.all(np.abs(lse - olse) <= 1e-4 * np.maximum(1, np.abs(olse)))
        assert np.all(np.abs(pmax - opmax) <= 1e-3 * np.maximum(1, np.abs(opmax)))
        # the oracle's combine on the GPU's summaries reproduces the GPU's combine
        # up to the last-ulp differences of the noise transform
        ref_g = oracle.group_combine(lse, pmax, arg, seed, step, oracle.GROUP_MODE_GUMBEL)
        diff = np.flatnonzero(ref_g != comb_g.cpu().numpy())
        for b in diff:
            keys = lse[:, b].astype(np.float64) + np.array(
                [oracle.gumbel32(oracle.group_noise_bits(seed, step, int(b), k)) for k in range(n_groups)])
            srt = np.sort(keys)[::-1]
            assert srt[0] - srt[1] < 1e-3 * (1 + abs(srt[0]))
        # arg equality with the oracle up to near-ties inside the group
        for k, b in np.argwhere(arg != oarg):
            p = oracle.perturbed_row(L[b], T, seed, step, int(b), mask_row=mask[b])
            assert p[oarg[k, b]] - p[arg[k, b]] < 1e-3 * (1 + abs(float(p[oarg[k, b]])))


@pytest.mark.parametrize("B,d,G,n_groups,path", [
    (6, 256, 512, 8, 0),      # more groups than one tile each would need
    (64, 768, 1024, 4, 0),    # four batch blocks
    (3, 520, 48, 9, 0),       # groups not a multiple of 32 ids (offsets cross mask words)
    (5, 4096, 2000, 3, 2),    # chunked H, forced MFMA path
    (24, 4096, 32768, 2, 0),  # chunk-outer kernel, 16 blocks a tile: XCD-weighted tiles in each group
])
def test_group_summaries_in_one_launch(fs, ctx, B, d, G, n_groups, path):
    # fs_group_summaries over consecutive groups equals the oracle's per-group
    # summaries (and hence fs_group_summary called group by group)
    import torch

    V = G * n_groups
    say(f"group summaries in one launch B={B} d={d} G={G} groups={n_groups} path={path}")
    H = synth.normal_bf16(B, d, seed=19)
    W = synth.normal_bf16(V, d, seed=20, std=1.5 / math.sqrt(d))
    allowed = np.random.default_rng(21).random((B, V)) >= 0.25
    allowed[1] = False
    mask = synth.pack_mask(allowed)
    L = oracle.logits(H, W)
    Hd, Wd, md = dev_bf16(H), dev_bf16(W), dev_words(mask)
    T, seed = 0.9, 78
    for step in range(3):
        summ = fs.fs_group_summaries(ctx, Hd, Wd, 0, G, T, seed, step, mask=md, path=path)
        flat = fs.fs_fmms_sample(ctx, Hd, Wd, T, seed, step, mask=md, path=path)
        comb_m = fs.fs_group_combine(ctx, summ, seed, step, fs.FS_COMBINE_MAX)
        _sync()
        assert torch.equal(comb_m, flat), "max-combine must equal the flat sample"
        lse, pmax, arg = (x.cpu().numpy() for x in fs.summary_views(summ))
        for k in range(n_groups):
            olse, opmax, oarg = oracle.group_summary(L, k * G, G, T, seed, step, mask=mask)
            fin = np.isfinite(olse)
            assert np.array_equal(fin, np.isfinite(lse[k])) and np.all(arg[k][~fin] == -1)
            assert np.all(np.abs(lse[k][fin] - olse[fin]) <= 1e-4 * np.maximum(1, np.abs(olse[fin])))
            assert np.all(np.abs(pmax[k][fin] - opmax[fin]) <= 1e-3 * np.maximum(1, np.abs(opmax[fin])))
            for b in np.flatnonzero(arg[k] != oarg):
                p = oracle.perturbed_row(L[b], T, seed, step, int(b), mask_row=mask[b])
                assert p[oarg[b]] - p[arg[k, b]] < 1e-3 * (1 + abs(float(p[oarg[b]])))


def test_group_summaries_match_group_by_group_calls(fs, ctx):
    import torch

    B, d, G, n_groups = 9, 512, 4096, 5
    H = synth.normal_bf16(B, d, seed=22)
    W = synth.normal_bf16(G * n_groups, d, seed=23, std=0.08)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    one = fs.fs_group_summaries(ctx, Hd, Wd, 32 * 7, G, 1.0, 5, 2)
    each = torch.empty_like(one)
    for k in range(n_groups):
        fs.fs_group_summary(ctx, Hd, Wd[k * G:(k + 1) * G], 32 * 7 + k * G, 1.0, 5, 2, out=each[k])
    _sync()
    # the two tilings may run different kernel forms (fp32 sums in another k
    # order), so maxima agree to rounding and ids up to near-ties
    a = [x.cpu().numpy() for x in fs.summary_views(one)]
    b = [x.cpu().numpy() for x in fs.summary_views(each)]
    assert np.allclose(a[0], b[0], rtol=1e-5, atol=1e-5)
    assert np.allclose(a[1], b[1], rtol=1e-5, atol=1e-5)
    diff = a[2] != b[2]
    assert diff.mean() <= 1e-3 + 1e-9 or np.all(np.abs(a[1][diff] - b[1][diff]) < 1e-3 * (1 + np.abs(b[1][diff])))


@pytest.mark.parametrize("B,d,V", [(100, 512, 3001), (128, 1024, 5000), (200, 512, 3001), (256, 512, 70001),
                                   (100, 256, 262143), (256, 256, 262143)])
def test_tile_maxima_wide(fs, ctx, B, d, V):
    # per-tile maximizers of the wide kernel (eight and sixteen batch blocks,
    # tiles of one pass and of four: 64 blocks a tile at V = 262143) against
    # the oracle's
    import torch

    H = synth.normal_bf16(B, d, seed=300 + B)
    W = synth.normal_bf16(V, d, seed=301, std=2.0 / math.sqrt(d))
    L = oracle.logits(H, W)
    nt, bounds = fs.fs_fmms_tiling(ctx, B, d, V, 0)
    say(f"tile maxima wide B={B} d={d} V={V} n_tiles={nt}")
    tmax = torch.empty((B, nt), dtype=torch.float32, device="cuda")
    targ = torch.empty((B, nt), dtype=torch.int32, device="cuda")
    fs.fs_fmms_sample(ctx, dev_bf16(H), dev_bf16(W), 0.8, 5, 3, tile_max=tmax, tile_arg=targ)
    _sync()
    omax, oarg = oracle.tile_maxima(L, 0.8, 5, 3, np.array(bounds))
    p_rows = [oracle.perturbed_row(L[b], 0.8, 5, 3, b) for b in range(B)]
    check_tiles(tmax.cpu().numpy(), targ.cpu().numpy(), omax, oarg, p_rows, bounds, f"wide tiles B={B}")
