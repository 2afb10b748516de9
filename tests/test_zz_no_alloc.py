"""The allocation-free entry point (fs_fmms_sample_noalloc) against fs_fmms_sample.

fs_fmms_sample_noalloc keeps its per-tile winners in the library's static
device array instead of a context's workspace.  Two calls in a row, the
second with a smaller input (the array keeps the first call's contents), must
each return what fs_fmms_sample returns for the same arguments; both are also
checked against the oracle under the near-tie rule.  Sizes past the array's
maximum are rejected before any launch.
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


def _case(B, d, V, seed, masked):
    H = synth.normal_bf16(B, d, seed=seed)
    W = synth.normal_bf16(V, d, seed=seed + 1, std=2.0 / np.sqrt(d))
    mask = None
    if masked:
        allowed = np.random.default_rng(seed + 2).random((B, V)) >= 0.3
        allowed[0] = False
        allowed[0, V - 1] = True  # a single allowed id, in the ragged tail
        mask = synth.pack_mask(allowed)
    return H, W, mask


def test_noalloc_matches_fmms_sample_two_calls(fs):
    import torch

    ctx = fs.fs_create(0, max_B=256, max_V=262144, max_top_k=0)
    try:
        # the second call is smaller than the first: fewer rows, tiles and ids
        for B, d, V, T, seed, masked in ((200, 2048, 70001, 0.8, 60, False), (7, 520, 3001, 1.1, 70, True)):
            say(f"no-alloc B={B} d={d} V={V} T={T} masked={masked}")
            H, W, mask = _case(B, d, V, seed, masked)
            Hd, Wd = dev_bf16(H), dev_bf16(W)
            md = None if mask is None else dev_words(mask)
            steps = range(4)
            got = torch.stack([fs.fs_fmms_sample_noalloc(Hd, Wd, T, 5, s, mask=md) for s in steps])
            ref = torch.stack([fs.fs_fmms_sample(ctx, Hd, Wd, T, 5, s, mask=md) for s in steps])
            torch.cuda.synchronize()
            got, ref = got.cpu().numpy(), ref.cpu().numpy()
            assert np.array_equal(got, ref), "the allocation-free call differs from fs_fmms_sample"
            L = oracle.logits(H, W)
            rows = np.arange(B)
            ora, _ = oracle.sample_rows_steps(L, rows, T, 5, 0, len(steps), mask=mask)
            n = check_ids(got, ora, oracle_p_fn(L, rows, T, 5, 0, mask=mask), f"no-alloc B={B}")
            say(f"  equal to fs_fmms_sample; {n} near-tie mismatches against the oracle")
            if masked:
                assert np.all(got[:, 0] == V - 1)
    finally:
        torch.cuda.synchronize()
        fs.fs_destroy(ctx)


def test_noalloc_rejects_sizes_past_the_scratch(fs):
    import torch

    H = dev_bf16(synth.normal_bf16(257, 256, seed=80))
    W = dev_bf16(synth.normal_bf16(1000, 256, seed=81, std=0.05))
    out = torch.full((257,), -7, dtype=torch.int32, device="cuda")
    lib = fs.binding._lib
    rc = lib.fs_fmms_sample_noalloc(None, H.data_ptr(), H.stride(0), W.data_ptr(), W.stride(0), 257, 256, 1000, 1.0,
                                    0, 0, None, 0, out.data_ptr())
    assert rc == fs.binding.FS_ERR_CAPACITY and "256" in fs.fs_last_error()
    rc = lib.fs_fmms_sample_noalloc(None, H.data_ptr(), H.stride(0), W.data_ptr(), W.stride(0), 0, 256, 1000, 1.0,
                                    0, 0, None, 0, out.data_ptr())
    assert rc == fs.binding.FS_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out == -7).item(), "a rejected call wrote its output"
