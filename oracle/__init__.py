"""CPU oracle for FlashSampling's fused LM-head matmul + sample.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It is a plain, slow
definition of what the sampler computes (see ``fs_oracle.c`` for the passages
it follows and the readings it takes) and shares no code with the HIP library.

This module is argument marshalling over ``libfsoracle.so`` (numpy in, numpy
out).  Arrays of bf16 values are carried as ``uint16`` bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

GROUP_MODE_GUMBEL = 0
GROUP_MODE_MAX = 1


def lib():
    """Load libfsoracle.so, compiling it first if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i64, u64, u32, i32, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float
        sig = {
            "fso_philox4x32_10": (None, [P, P, P]),
            "fso_noise_bits": (u32, [u64, u64, u32, u32]),
            "fso_group_noise_bits": (u32, [u64, u64, u32, u32]),
            "fso_gumbel64": (ctypes.c_double, [u32]),
            "fso_gumbel32": (f32, [u32]),
            "fso_gumbel32_range": (None, [u64, i64, P]),
            "fso_gumbel_scan": (None, [u64, u64, P, P]),
            "fso_logits": (None, [P, i64, P, i64, i32, i32, i64, P]),
            "fso_logits_fp32acc": (None, [P, i64, P, i64, i32, i32, i64, P]),
            "fso_scores_row": (None, [P, i64, f32, P, i32, f32, P]),
            "fso_perturbed_row": (None, [P, i64, f32, u64, u64, i32, P, i32, f32, P]),
            "fso_argmax": (i64, [P, i64]),
            "fso_sample_from_logits": (None, [P, i32, i64, f32, u64, u64, P, i64, i32, f32, P, P]),
            "fso_sample_steps": (None, [P, i32, i64, f32, u64, u64, i64, P, i64, i32, f32, P]),
            "fso_sample_rows_steps": (None, [P, P, i32, i64, f32, u64, u64, i64, P, i64, i32, f32, P, P]),
            "fso_tile_maxima": (None, [P, i32, i64, f32, u64, u64, P, i64, P, i32, P, P]),
            "fso_group_summary": (None, [P, i32, i64, i64, i64, f32, u64, u64, P, i64, P, P, P]),
            "fso_group_combine": (None, [P, P, P, i32, i32, u64, u64, i32, P]),
            "fso_grouped_sample_steps": (None, [P, i32, i64, f32, u64, u64, i64, P, i64, P, i32, i32, P]),
            "fso_fmms_sample": (None, [P, i64, P, i64, i32, i32, i64, f32, u64, u64, P, i64, i32, f32, P]),
            "fso_num_threads": (i32, []),
            "fso_uniform_bits": (u32, [u64, u64, u32]),
            "fso_uniform64": (ctypes.c_double, [u32]),
            "fso_cdf_sample_row": (i64, [P, i64, f32, P, ctypes.c_double]),
            "fso_cdf_sample_rows_steps": (None, [P, P, i32, i64, f32, u64, u64, i32, P, i64, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().fso_num_threads()


# --- noise -----------------------------------------------------------------

def philox4x32_10(key, ctr):
    """One Philox4x32-10 block: key (2 words), counter (4 words) -> 4 words."""
    k = _c(key, np.uint32)
    c = _c(ctr, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().fso_philox4x32_10(_ptr(k), _ptr(c), _ptr(out))
    return out


def noise_bits(seed: int, step: int, row: int, v: int) -> int:
    return int(lib().fso_noise_bits(seed, step, row, v))


def noise_bits_range(seed: int, step: int, row: int, v0: int, n: int) -> np.ndarray:
    f = lib().fso_noise_bits
    return np.array([f(seed, step, row, v) for v in range(v0, v0 + n)], np.uint32)


def group_noise_bits(seed: int, step: int, row: int, k: int) -> int:
    return int(lib().fso_group_noise_bits(seed, step, row, k))


def gumbel64(r: int) -> float:
    return float(lib().fso_gumbel64(r))


def gumbel32(r: int) -> float:
    return float(lib().fso_gumbel32(r))


def gumbel32_range(r0: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().fso_gumbel32_range(r0, n, _ptr(out))
    return out


def gumbel_scan(r_lo: int = 0, r_hi: int = 1 << 32):
    """(nonfinite count, decrease count, min, max) of fp32 noise over words [r_lo, r_hi)."""
    stats = np.zeros(2, np.int64)
    mm = np.zeros(2, np.float64)
    lib().fso_gumbel_scan(r_lo, r_hi, _ptr(stats), _ptr(mm))
    return int(stats[0]), int(stats[1]), float(mm[0]), float(mm[1])


# --- logits and sampling -----------------------------------------------------

def logits(H, W, fp32_acc: bool = False) -> np.ndarray:
    """[B, V] fp32 logits of bf16 H [B, d] and W [V, d] (uint16 bit patterns)."""
    H = _c(H, np.uint16)
    W = _c(W, np.uint16)
    B, d = H.shape
    V, d2 = W.shape
    assert d == d2
    out = np.empty((B, V), np.float32)
    fn = lib().fso_logits_fp32acc if fp32_acc else lib().fso_logits
    fn(_ptr(H), d, _ptr(W), d, B, d, V, _ptr(out))
    return out


def _mask_args(mask, B):
    if mask is None:
        return None, 0
    m = _c(mask, np.uint32)
    assert m.ndim == 2 and m.shape[0] == B
    return m, m.shape[1]


def scores_row(logit_row, T, mask_row=None, top_k=0, top_p=1.0):
    x = _c(logit_row, np.float32)
    m = None if mask_row is None else _c(mask_row, np.uint32)
    out = np.empty_like(x)
    lib().fso_scores_row(_ptr(x), x.shape[0], T, _ptr(m), top_k, top_p, _ptr(out))
    return out


def perturbed_row(logit_row, T, seed, step, row, mask_row=None, top_k=0, top_p=1.0):
    x = _c(logit_row, np.float32)
    m = None if mask_row is None else _c(mask_row, np.uint32)
    out = np.empty_like(x)
    lib().fso_perturbed_row(_ptr(x), x.shape[0], T, seed, step, row, _ptr(m), top_k, top_p, _ptr(out))
    return out


def argmax(p) -> int:
    p = _c(p, np.float32)
    return int(lib().fso_argmax(_ptr(p), p.shape[0]))


def sample_from_logits(L, T, seed, step, mask=None, top_k=0, want_p=False, top_p=1.0):
    """One step: returns out_idx [B] (int32) and, if asked, p [B, V]."""
    L = _c(L, np.float32)
    B, V = L.shape
    m, ldm = _mask_args(mask, B)
    out = np.empty(B, np.int32)
    p = np.empty((B, V), np.float32) if want_p else None
    lib().fso_sample_from_logits(_ptr(L), B, V, T, seed, step, _ptr(m), ldm, top_k, top_p, _ptr(out), _ptr(p))
    return (out, p) if want_p else out


def sample_steps(L, T, seed, step0, nsteps, mask=None, top_k=0, top_p=1.0):
    """[nsteps, B] samples for steps step0 .. step0 + nsteps - 1."""
    L = _c(L, np.float32)
    B, V = L.shape
    m, ldm = _mask_args(mask, B)
    out = np.empty((nsteps, B), np.int32)
    lib().fso_sample_steps(_ptr(L), B, V, T, seed, step0, nsteps, _ptr(m), ldm, top_k, top_p, _ptr(out))
    return out


def uniform_bits(seed: int, step: int, row: int) -> int:
    return int(lib().fso_uniform_bits(seed, step, row))


def uniform64(r: int) -> float:
    return float(lib().fso_uniform64(r))


def cdf_sample_row(logit_row, T, u, mask_row=None) -> int:
    x = _c(logit_row, np.float32)
    m = None if mask_row is None else _c(mask_row, np.uint32)
    return int(lib().fso_cdf_sample_row(_ptr(x), x.shape[0], T, _ptr(m), u))


def cdf_sample_rows_steps(L, rows, T, seed, step0, nsteps, mask=None):
    """Conventional comparator: (ids, u), each [nsteps, R]."""
    L = _c(L, np.float32)
    R, V = L.shape
    rows = _c(rows, np.int32)
    m = None if mask is None else _c(mask, np.uint32)
    ldm = 0 if m is None else m.shape[1]
    ids = np.empty((nsteps, R), np.int32)
    u = np.empty((nsteps, R), np.float64)
    lib().fso_cdf_sample_rows_steps(_ptr(L), _ptr(rows), R, V, T, seed, step0, nsteps, _ptr(m), ldm, _ptr(ids),
                                    _ptr(u))
    return ids, u


def sample_rows_steps(L, rows, T, seed, step0, nsteps, mask=None, top_k=0, top_p=1.0):
    """Samples of global rows `rows` (logits L[i] belong to row rows[i]) for nsteps steps.

    Returns (ids, pmax), each [nsteps, R].  mask, if given, is the full [B, ldm] mask.
    """
    L = _c(L, np.float32)
    R, V = L.shape
    rows = _c(rows, np.int32)
    assert rows.shape == (R,)
    m = None if mask is None else _c(mask, np.uint32)
    ldm = 0 if m is None else m.shape[1]
    ids = np.empty((nsteps, R), np.int32)
    pmax = np.empty((nsteps, R), np.float32)
    lib().fso_sample_rows_steps(_ptr(L), _ptr(rows), R, V, T, seed, step0, nsteps, _ptr(m), ldm, top_k, top_p,
                                _ptr(ids),
                                _ptr(pmax))
    return ids, pmax


def tile_maxima(L, T, seed, step, bounds, mask=None):
    L = _c(L, np.float32)
    B, V = L.shape
    m, ldm = _mask_args(mask, B)
    bnd = _c(bounds, np.int64)
    n = bnd.shape[0] - 1
    tmax = np.empty((B, n), np.float32)
    targ = np.empty((B, n), np.int32)
    lib().fso_tile_maxima(_ptr(L), B, V, T, seed, step, _ptr(m), ldm, _ptr(bnd), n, _ptr(tmax), _ptr(targ))
    return tmax, targ


def group_summary(L, vocab_offset, G, T, seed, step, mask=None):
    """(lse, pmax, arg) [B] each for group [vocab_offset, vocab_offset + G)."""
    L = _c(L, np.float32)
    B, V = L.shape
    m, ldm = _mask_args(mask, B)
    lse = np.empty(B, np.float32)
    pmax = np.empty(B, np.float32)
    arg = np.empty(B, np.int32)
    lib().fso_group_summary(_ptr(L), B, V, vocab_offset, G, T, seed, step, _ptr(m), ldm, _ptr(lse), _ptr(pmax),
                            _ptr(arg))
    return lse, pmax, arg


def group_combine(lse, pmax, arg, seed, step, mode):
    """Combine [n_groups, B] summaries into [B] samples."""
    lse = _c(lse, np.float32)
    pmax = _c(pmax, np.float32)
    arg = _c(arg, np.int32)
    n_groups, B = lse.shape
    out = np.empty(B, np.int32)
    lib().fso_group_combine(_ptr(lse), _ptr(pmax), _ptr(arg), n_groups, B, seed, step, mode, _ptr(out))
    return out


def grouped_sample_steps(L, T, seed, step0, nsteps, bounds, mode, mask=None):
    L = _c(L, np.float32)
    B, V = L.shape
    m, ldm = _mask_args(mask, B)
    bnd = _c(bounds, np.int64)
    out = np.empty((nsteps, B), np.int32)
    lib().fso_grouped_sample_steps(_ptr(L), B, V, T, seed, step0, nsteps, _ptr(m), ldm, _ptr(bnd),
                                   bnd.shape[0] - 1, mode, _ptr(out))
    return out


def fmms_sample(H, W, T, seed, step, mask=None, top_k=0, top_p=1.0):
    """End to end from bf16 operands: [B] sampled ids."""
    H = _c(H, np.uint16)
    W = _c(W, np.uint16)
    B, d = H.shape
    V = W.shape[0]
    m, ldm = _mask_args(mask, B)
    out = np.empty(B, np.int32)
    lib().fso_fmms_sample(_ptr(H), d, _ptr(W), d, B, d, V, T, seed, step, _ptr(m), ldm, top_k, top_p, _ptr(out))
    return out
