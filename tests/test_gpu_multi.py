"""GPU parity of several samples per row from one pass over W.

fs_fmms_sample_multi(num_samples = S) draws, for row b, the ids that
fs_fmms_sample would return at steps step, step + 1, ..., step + S - 1: the
oracle checks them as S ordinary steps.  Cases: virtual batches (rows x
samples) inside one 16-row block, across batch blocks, and across the 64-row
launch chunks (a row's samples split between two launches); masks; the
dot-product path; steps that carry into the upper 32 bits; S = 1.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_ids, dev_bf16, dev_words, oracle_p_fn, say

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

    c = fs.fs_create(0, max_B=64, max_V=262144, max_top_k=0)
    torch.cuda.synchronize()
    yield c
    torch.cuda.synchronize()
    fs.fs_destroy(c)


def _check_multi(fs, ctx, H, W, T, seed, step, S, mask=None, path=0, calls=2, label=""):
    import torch

    B = H.shape[0]
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    md = None if mask is None else dev_words(mask)
    L = oracle.logits(H, W)
    rows = np.arange(B)
    for c in range(calls):
        st = step + c * S
        got = fs.fs_fmms_sample_multi(ctx, Hd, Wd, T, seed, st, S, mask=md, path=path)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        assert got.shape == (B, S)
        want, _ = oracle.sample_rows_steps(L, rows, T, seed, st, S, mask=mask)  # [S, B]
        n = check_ids(got.T, want, oracle_p_fn(L, rows, T, seed, st, mask=mask), label)
        say(f"{label} call {c}: {n} near-tie mismatches over {got.size} draws")
    return L


@pytest.mark.parametrize("B,d,V,S,path", [
    (3, 256, 4096, 4, 0),      # 12 virtual rows: one 16-row block
    (5, 520, 3000, 7, 0),      # 35: three blocks, general driver (d % 256 != 0)
    (7, 4096, 5000, 6, 0),     # 42 virtual rows with chunked H
    (20, 256, 2000, 5, 0),     # 100: two launches, row 12's samples split between them
    (1, 512, 1500, 2, 1),      # dot-product path
    (2, 768, 999, 33, 2),      # 66 virtual rows, forced MFMA path
    (6, 4096, 65551, 4, 0),    # 24 virtual rows, chunk-outer kernel with XCD-weighted tiles
])
def test_multi_sample_parity(fs, ctx, B, d, V, S, path):
    say(f"multi-sample B={B} d={d} V={V} S={S} path={path}")
    H = synth.normal_bf16(B, d, seed=61 + B)
    W = synth.normal_bf16(V, d, seed=62 + V, std=2.0 / np.sqrt(d))
    _check_multi(fs, ctx, H, W, 0.8, 11, 5, S, path=path, label=f"multi {B}x{S}")


def test_multi_sample_one_equals_single(fs, ctx):
    import torch

    B, d, V = 9, 512, 2000
    H = synth.normal_bf16(B, d, seed=71)
    W = synth.normal_bf16(V, d, seed=72, std=0.05)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    for step in (0, 3):
        a = fs.fs_fmms_sample_multi(ctx, Hd, Wd, 1.0, 2, step, 1)
        b = fs.fs_fmms_sample(ctx, Hd, Wd, 1.0, 2, step)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy()[:, 0], b.cpu().numpy())


def test_multi_sample_step_carry(fs, ctx):
    # steps 2^32 - 2 .. 2^32 + 1: the low word wraps and the high word carries
    B, d, V, S = 4, 256, 3000, 4
    H = synth.normal_bf16(B, d, seed=73)
    W = synth.normal_bf16(V, d, seed=74, std=0.1)
    _check_multi(fs, ctx, H, W, 1.0, 5, (1 << 32) - 2, S, calls=1, label="step carry")


def test_multi_sample_masked(fs, ctx):
    B, d, V, S = 6, 520, 3000, 5
    H = synth.normal_bf16(B, d, seed=75)
    W = synth.outlier_bf16(V, d, 76, 77, 0.05, 0.5, 0.01)
    allowed = np.random.default_rng(78).random((B, V)) >= 0.3
    allowed[1] = False
    allowed[4] = False
    allowed[4, [7, 2500]] = True
    mask = synth.pack_mask(allowed)
    _check_multi(fs, ctx, H, W, 1.0, 9, 0, S, mask=mask, label="masked multi")


def test_multi_sample_rejects_bad_counts(fs, ctx):
    B, d, V = 2, 256, 500
    Hd = dev_bf16(synth.normal_bf16(B, d, seed=79))
    Wd = dev_bf16(synth.normal_bf16(V, d, seed=80))
    with pytest.raises(fs.FSError):
        fs.fs_fmms_sample_multi(ctx, Hd, Wd, 1.0, 0, 0, 0)
