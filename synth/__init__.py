"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds no part of the sampler's arithmetic: it only draws operands
(hidden states H, LM-head weights W, vocabulary masks) from fixed seeds, rounds
them to bf16 and packs masks into the words the library reads.  Both sides of
every parity check take their inputs from here.

Shapes and distributions follow the decode-head workloads the sampler is
measured on (vocabulary 151936, the "~150k words" scale of the pages; model
dimensions 2048 / 4096 / 5120 / 7168).  No trained weights or datasets are
used; every value is drawn from numpy's PCG64 generator.

Recipe (seeds per workload index c):
  H = N(0, 1)                 seed 1000 c + 1
  W = N(0, std^2)             seed 1000 c + 2   (std 1/sqrt(d) for the tiny case,
                                                 0.02 for the decode heads)
  W outliers (masked case)    seed 1000 c + 4   (each element N(0, 0.2^2) with
                                                 probability 0.01)
  mask (masked case)          seed 1000 c + 3   (each id disallowed with
                                                 probability 0.3, >= 1 allowed)
Large arrays are drawn in fixed blocks of rows, each from its own
SeedSequence([seed, block]), so the result does not depend on thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_ROWS = 2048


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_rng(seed: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block])))


def _fill_blocks(rows: int, cols: int, fill) -> np.ndarray:
    out = np.empty((rows, cols), np.uint16)
    n_blocks = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def work(i):
        r0 = i * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        out[r0:r1] = fill(i, r1 - r0)

    if n_blocks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_blocks)))
    return out


def normal_bf16(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """[rows, cols] bf16 bit patterns of N(0, std^2) drawn in fp32."""
    def fill(i, n):
        z = _block_rng(seed, i).standard_normal((n, cols), dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        return bf16_round(z)

    return _fill_blocks(rows, cols, fill)


def outlier_bf16(rows: int, cols: int, seed: int, seed_outlier: int, std: float, std_out: float,
                 p_out: float) -> np.ndarray:
    """N(0, std^2) with each element replaced by N(0, std_out^2) with probability p_out."""
    def fill(i, n):
        z = _block_rng(seed, i).standard_normal((n, cols), dtype=np.float32)
        flag = _block_rng(seed_outlier, i).random((n, cols), dtype=np.float32) < np.float32(p_out)
        scale = np.where(flag, np.float32(std_out), np.float32(std))
        return bf16_round(z * scale)

    return _fill_blocks(rows, cols, fill)


def small_int_bf16(rows: int, cols: int, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Integers in [lo, hi] as bf16 (exact); sums of their products are exact in fp32 for small d."""
    z = np.random.default_rng(seed).integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)
    return bf16_round(z)


def mask_words(V: int) -> int:
    return (V + 31) // 32


def pack_mask(allowed: np.ndarray) -> np.ndarray:
    """bool [B, V] -> uint32 [B, ceil(V/32)]: bit (v & 31) of word (v >> 5) set when v is allowed."""
    allowed = np.asarray(allowed, dtype=bool)
    B, V = allowed.shape
    nw = mask_words(V)
    padded = np.zeros((B, nw * 32), dtype=bool)
    padded[:, :V] = allowed
    bits = padded.reshape(B, nw, 32).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=2).astype(np.uint32)


def unpack_mask(words: np.ndarray, V: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    B = words.shape[0]
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return bits.reshape(B, -1)[:, :V].astype(bool)


def bernoulli_mask(B: int, V: int, seed: int, p_disallow: float = 0.3) -> np.ndarray:
    """Packed mask with each id disallowed with probability p_disallow; every row keeps >= 1 id."""
    rng = np.random.default_rng(seed)
    allowed = rng.random((B, V), dtype=np.float32) >= np.float32(p_disallow)
    empty = ~allowed.any(axis=1)
    allowed[empty, 0] = True
    return pack_mask(allowed)


# --- the workloads -----------------------------------------------------------

V_DECODE = 151936  # decode-head vocabulary

WORKLOADS = {
    # index c, default shapes, temperature, W std, B values
    "tiny": dict(c=0, B=4, d=256, V=4096, T=1.0, w_std=None, Bs=[4]),
    "small_decode": dict(c=1, B=64, d=2048, V=V_DECODE, T=1.0, w_std=0.02, Bs=[1, 2, 4, 8, 16, 32, 64]),
    "mid_decode": dict(c=2, B=64, d=4096, V=V_DECODE, T=0.7, w_std=0.02, Bs=[1, 8, 32, 64, 128, 256], top_k=50),
    "masked": dict(c=3, B=32, d=5120, V=V_DECODE, T=1.0, w_std=0.02, Bs=[32]),
    "grouped": dict(c=4, B=64, d=7168, V=262144, T=1.0, w_std=0.02, Bs=[64], n_groups=8),
}


def workload_H(name: str, B: int | None = None, d: int | None = None) -> np.ndarray:
    w = WORKLOADS[name]
    B = w["B"] if B is None else B
    d = w["d"] if d is None else d
    z = np.random.default_rng(1000 * w["c"] + 1).standard_normal((B, d), dtype=np.float32)
    return bf16_round(z)


def workload_W(name: str, V: int | None = None, d: int | None = None) -> np.ndarray:
    w = WORKLOADS[name]
    V = w["V"] if V is None else V
    d = w["d"] if d is None else d
    c = w["c"]
    std = w["w_std"] if w["w_std"] is not None else 1.0 / np.sqrt(d)
    if name == "masked":
        return outlier_bf16(V, d, 1000 * c + 2, 1000 * c + 4, std, 0.2, 0.01)
    return normal_bf16(V, d, 1000 * c + 2, std)


def workload_mask(name: str, B: int | None = None, V: int | None = None) -> np.ndarray | None:
    w = WORKLOADS[name]
    if name != "masked":
        return None
    B = w["B"] if B is None else B
    V = w["V"] if V is None else V
    return bernoulli_mask(B, V, 1000 * w["c"] + 3, 0.3)


def group_bounds(V: int, n_groups: int) -> np.ndarray:
    """Contiguous equal groups over [0, V) (V divisible by n_groups)."""
    assert V % n_groups == 0
    G = V // n_groups
    return np.arange(n_groups + 1, dtype=np.int64) * G
