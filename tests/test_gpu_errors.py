"""Argument checks of the sampling entry points on a live context.

Every call below breaks one documented precondition of include/flashsampling.h
and must return its error code with a message, enqueue nothing (the output
buffer keeps its sentinel) and leave the context usable: a valid call after
all of them still matches the oracle.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_ids, dev_bf16, oracle_p_fn, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import lm_head_matmul_amd as fs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ctx = fs.fs_create(0, max_B=16, max_V=8192, max_top_k=8)
    torch.cuda.synchronize()
    yield fs, ctx
    torch.cuda.synchronize()
    fs.fs_destroy(ctx)


def _bufs(B=4, d=256, V=1000):
    import torch

    H = dev_bf16(synth.normal_bf16(B, d, seed=41))
    W = dev_bf16(synth.normal_bf16(V, d, seed=42, std=0.05))
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    return H, W, out


def _sample_call(fs, ctx, Ht, Wt, outt, **kw):
    """fs_fmms_sample through the C ABI with every argument overridable."""
    a = dict(stream=None, H=Ht.data_ptr(), ldh=Ht.stride(0), W=Wt.data_ptr(), ldw=Wt.stride(0), B=Ht.shape[0],
             d=Ht.shape[1], V=Wt.shape[0], T=1.0, seed=1, step=2, mask=None, ldm=0, top_k=0, out=outt.data_ptr(),
             tmax=None, targ=None, path=0)
    a.update(kw)
    return fs.binding._lib.fs_fmms_sample(ctx, a["stream"], a["H"], a["ldh"], a["W"], a["ldw"], a["B"], a["d"],
                                          a["V"], a["T"], a["seed"], a["step"], a["mask"], a["ldm"], a["top_k"],
                                          a["out"], a["tmax"], a["targ"], a["path"])


SAMPLE_CASES = [
    ("B = 0", dict(B=0), -1),
    ("B > max_B", dict(B=17), -3),
    ("d not a multiple of 8", dict(d=250), -1),
    ("ldh < d", dict(ldh=128), -1),
    ("ldw not a multiple of 8", dict(ldw=260), -1),
    ("H misaligned", "H+2", -1),
    ("W misaligned", "W+8", -1),
    ("V = 0", dict(V=0), -1),
    ("V > max_V", dict(V=8193), -3),
    ("T = 0", dict(T=0.0), -1),
    ("T < 0", dict(T=-1.0), -1),
    ("T = inf", dict(T=float("inf")), -1),
    ("T = nan", dict(T=float("nan")), -1),
    ("top_k < 0", dict(top_k=-1), -1),
    ("top_k > max_top_k", dict(top_k=9), -3),
    ("unknown path", dict(path=3), -1),
    ("dot path with B > 2", dict(path=1), -2),
    ("out is NULL", dict(out=None), -1),
    ("H is NULL", dict(H=None), -1),
]


@pytest.mark.parametrize("label,change,code", SAMPLE_CASES, ids=[c[0] for c in SAMPLE_CASES])
def test_fmms_sample_rejects(env, label, change, code):
    import torch

    fs, ctx = env
    say(f"argument check: {label}")
    H, W, out = _bufs()
    if change == "H+2":
        kw = dict(H=H.data_ptr() + 2)
    elif change == "W+8":
        kw = dict(W=W.data_ptr() + 8)
    else:
        kw = change
    rc = _sample_call(fs, ctx, H, W, out, **kw)
    torch.cuda.synchronize()
    assert rc == code, f"{label}: got {rc}, message {fs.fs_last_error()!r}"
    assert fs.fs_last_error(), "an error must come with a message"
    assert torch.all(out == -7).item(), f"{label}: the call wrote its output"


def test_mask_stride_and_tile_arguments(env):
    import torch

    fs, ctx = env
    H, W, out = _bufs(V=1000)
    mask = torch.full((4, 31), -1, dtype=torch.int32, device="cuda")  # ceil(1000/32) = 32 words needed
    rc = _sample_call(fs, ctx, H, W, out, mask=mask.data_ptr(), ldm=31)
    assert rc == -1
    n, _ = fs.fs_fmms_tiling(ctx, 4, 256, 1000)
    tmax = torch.empty((4, n), dtype=torch.float32, device="cuda")
    targ = torch.empty((4, n), dtype=torch.int32, device="cuda")
    assert _sample_call(fs, ctx, H, W, out, tmax=tmax.data_ptr()) == -1  # tile_max without tile_arg
    assert _sample_call(fs, ctx, H, W, out, tmax=tmax.data_ptr(), targ=targ.data_ptr(), top_k=3) == -1
    torch.cuda.synchronize()
    assert torch.all(out == -7).item()


def test_unfused_and_group_argument_checks(env):
    import torch

    fs, ctx = env
    lib = fs.binding._lib
    H, W, out = _bufs(V=1000)
    ws = torch.empty((4, 1004), dtype=torch.float32, device="cuda")
    base = (ctx, None, H.data_ptr(), H.stride(0), W.data_ptr(), W.stride(0), 4, 256, 1000, 1.0, 0, 0, None, 0, 0,
            out.data_ptr())
    assert lib.fs_unfused_sample(*base, ws.data_ptr(), 998, 0) == -1   # ldl < V
    assert lib.fs_unfused_sample(*base, ws.data_ptr(), 1002, 0) == -1  # ldl not a multiple of 4
    assert lib.fs_unfused_sample(*base, ws.data_ptr() + 4, 1004, 0) == -1  # misaligned workspace
    assert lib.fs_unfused_sample(*base, None, 1004, 0) == -1
    summ = torch.empty((4, 3), dtype=torch.int32, device="cuda")
    gargs = lambda off, G: (ctx, None, H.data_ptr(), H.stride(0), W.data_ptr(), W.stride(0), 4, 256, off, G, 1.0,  # noqa: E731
                            0, 0, None, 0, summ.data_ptr(), 0)
    assert lib.fs_group_summary(*gargs(16, 512)) == -1          # offset not a multiple of 32
    assert lib.fs_group_summary(*gargs(-32, 512)) == -1
    assert lib.fs_group_summary(*gargs((1 << 31) - 256, 512)) == -1  # past 2^31 ids
    s = torch.zeros((2, 4, 3), dtype=torch.int32, device="cuda")
    assert lib.fs_group_combine(ctx, None, s.data_ptr(), 0, 4, 0, 0, 0, out.data_ptr()) == -1
    assert lib.fs_group_combine(ctx, None, s.data_ptr(), 4097, 4, 0, 0, 0, out.data_ptr()) == -1
    assert lib.fs_group_combine(ctx, None, s.data_ptr(), 2, 4, 0, 0, 2, out.data_ptr()) == -1
    assert lib.fs_group_combine(ctx, None, s.data_ptr(), 2, 0, 0, 0, 0, out.data_ptr()) == -1
    n = ctypes.c_int64()
    assert lib.fs_fmms_tiling(ctx, 4, 256, 0, 0, ctypes.byref(n), None) == -1
    torch.cuda.synchronize()
    assert torch.all(out == -7).item()


def test_context_still_samples_after_errors(env):
    import torch

    fs, ctx = env
    Hh = synth.normal_bf16(4, 256, seed=41)
    Wh = synth.normal_bf16(1000, 256, seed=42, std=0.05)
    H, W, out = dev_bf16(Hh), dev_bf16(Wh), torch.empty(4, dtype=torch.int32, device="cuda")
    assert _sample_call(fs, ctx, H, W, out, T=0.0) == -1
    got = fs.fs_fmms_sample(ctx, H, W, 1.0, 1, 2, out=out).cpu().numpy()
    L = oracle.logits(Hh, Wh)
    rows = np.arange(4)
    want, _ = oracle.sample_rows_steps(L, rows, 1.0, 1, 2, 1)
    check_ids(got[None, :], want, oracle_p_fn(L, rows, 1.0, 1, 2), "after errors")


def test_binding_rejects_bad_buffers_before_any_launch(env):
    # the Python binding checks every output, workspace and mask tensor's dtype,
    # device, layout and size, and raises before the library is called
    import torch

    fs, ctx = env
    H, W, out = _bufs(V=1000)
    n, _ = fs.fs_fmms_tiling(ctx, 4, 256, 1000)
    bad_calls = {
        "out int64": lambda: fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, out=torch.zeros(4, dtype=torch.int64,
                                                                                     device="cuda")),
        "out too short": lambda: fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, out=out[:3]),
        "out on the host": lambda: fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, out=torch.zeros(4, dtype=torch.int32)),
        "out strided": lambda: fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0,
                                                 out=torch.zeros(8, dtype=torch.int32, device="cuda")[::2]),
        "tile_max too small": lambda: fs.fs_fmms_sample(
            ctx, H, W, 1.0, 0, 0, out=out, tile_max=torch.zeros((4, n - 1), device="cuda"),
            tile_arg=torch.zeros((4, n), dtype=torch.int32, device="cuda")),
        "tile_arg float": lambda: fs.fs_fmms_sample(
            ctx, H, W, 1.0, 0, 0, out=out, tile_max=torch.zeros((4, n), device="cuda"),
            tile_arg=torch.zeros((4, n), device="cuda")),
        "mask rows < B": lambda: fs.fs_fmms_sample(ctx, H, W, 1.0, 0, 0, out=out,
                                                   mask=torch.full((3, 32), -1, dtype=torch.int32, device="cuda")),
        "mask words < ceil(V/32)": lambda: fs.fs_fmms_sample(
            ctx, H, W, 1.0, 0, 0, out=out, mask=torch.full((4, 31), -1, dtype=torch.int32, device="cuda")),
        "logits_ws rows < B": lambda: fs.fs_unfused_sample(ctx, H, W, 1.0, 0, 0, out=out,
                                                            logits_ws=torch.zeros((3, 1000), device="cuda")),
        "logits_ws cols < V": lambda: fs.fs_softmax_sample(ctx, H, W, 1.0, 0, 0, out=out,
                                                           logits_ws=torch.zeros((4, 996), device="cuda")),
        "group out too short": lambda: fs.fs_group_summary(ctx, H, W[:512], 0, 1.0, 0, 0,
                                                           out=torch.zeros((3, 3), dtype=torch.int32, device="cuda")),
        "combine out too short": lambda: fs.fs_group_combine(
            ctx, torch.zeros((2, 4, 3), dtype=torch.int32, device="cuda"), 0, 0, out=out[:2]),
        "multi out too short": lambda: fs.fs_fmms_sample_multi(
            ctx, H, W, 1.0, 0, 0, 2, out=torch.zeros(7, dtype=torch.int32, device="cuda")),
    }
    for label, call in bad_calls.items():
        say(f"binding check: {label}")
        with pytest.raises((TypeError, ValueError)):
            call()
    torch.cuda.synchronize()
    assert torch.all(out == -7).item(), "a rejected call wrote its output"
