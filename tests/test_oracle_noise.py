"""Pins of the oracle's noise: Philox words and the uniform -> Gumbel transform.

The noise is a Philox counter generator keyed by a master seed and the
element's coordinates, mapped to a uniform u = (r+1)/(2^32+1) and to Gumbel
noise -log(-log u) [readus.org FlashSampling summary, code guide sections 2
(RNG) and 3 (floating point)].  These tests tie the oracle to things outside
itself: an independent Philox implementation (PyTorch's PhiloxRNGEngine.h,
written from the same SC'11 paper), 50-digit decimal arithmetic for the
transform, and the Gumbel distribution's closed forms.
"""
import math
import os
import shutil
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle

# --- Philox against an independent implementation ---------------------------

_ENGINE_SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
#include <cinttypes>
// stdin: lines "seed subsequence offset nwords"; stdout: the first nwords words.
int main() {
  unsigned long long seed, sub, off; int n;
  while (std::scanf("%llu %llu %llu %d", &seed, &sub, &off, &n) == 4) {
    at::philox_engine e(seed, sub, off);
    for (int i = 0; i < n; ++i) std::printf("%u%c", e(), i + 1 == n ? '\n' : ' ');
  }
  return 0;
}
"""


def _torch_include():
    try:
        import torch
    except Exception:
        return None
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    return inc if os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")) else None


@pytest.fixture(scope="module")
def torch_philox():
    inc = _torch_include()
    cxx = shutil.which("g++")
    if inc is None or cxx is None:
        pytest.skip("PyTorch's PhiloxRNGEngine.h or g++ not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "engine.cpp")
    exe = os.path.join(d, "engine")
    with open(src, "w") as f:
        f.write(_ENGINE_SRC)
    subprocess.run([cxx, "-O1", "-std=c++17", "-I", inc, src, "-o", exe], check=True)

    def run(queries):
        text = "".join(f"{s} {sub} {off} {n}\n" for s, sub, off, n in queries)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]

    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_block_matches_independent_engine(torch_philox):
    # PyTorch's engine: key = seed, counter = (offset lo, offset hi, subsequence lo, subsequence hi);
    # its first four draws are the four output words of that counter block.
    rng = np.random.default_rng(7)
    queries, blocks = [], []
    for _ in range(200):
        seed = int(rng.integers(0, 2**64, dtype=np.uint64))
        sub = int(rng.integers(0, 2**64, dtype=np.uint64))
        off = int(rng.integers(0, 2**64, dtype=np.uint64))
        queries.append((seed, sub, off, 4))
        key = [seed & 0xFFFFFFFF, seed >> 32]
        ctr = [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]
        blocks.append(oracle.philox4x32_10(key, ctr).tolist())
    # edge counters: all-zero, all-ones
    for seed, sub, off in [(0, 0, 0), (2**64 - 1, 2**64 - 1, 2**64 - 1), (0, 0, 1)]:
        queries.append((seed, sub, off, 4))
        blocks.append(oracle.philox4x32_10([seed & 0xFFFFFFFF, seed >> 32],
                                           [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]).tolist())
    ref = torch_philox(queries)
    assert ref == blocks


def test_noise_word_mapping_matches_independent_engine(torch_philox):
    # Reading of the keying: counter = (v >> 2, row, step lo, step hi), word v & 3.
    # In the engine's terms: subsequence = step, offset = (row << 32) | (v >> 2).
    rng = np.random.default_rng(11)
    cases, queries = [], []
    for _ in range(300):
        seed = int(rng.integers(0, 2**64, dtype=np.uint64))
        step = int(rng.integers(0, 2**40))
        row = int(rng.integers(0, 4096))
        v = int(rng.integers(0, 2**31 - 1))
        cases.append((seed, step, row, v))
        queries.append((seed, step, (row << 32) | (v >> 2), (v & 3) + 1))
    ref = torch_philox(queries)
    for (seed, step, row, v), words in zip(cases, ref):
        assert oracle.noise_bits(seed, step, row, v) == words[-1]


def test_group_noise_is_outside_vocab_counter_range():
    # Group noise uses counter word 0 = 0x40000000 | k; vocabulary ids v < 2^31 use v >> 2 < 2^29.
    for seed, step, row, k in [(0, 0, 0, 0), (5, 9, 3, 7), (2**63, 2**33, 17, 255)]:
        key = [seed & 0xFFFFFFFF, seed >> 32]
        ctr = [0x40000000 | k, row, step & 0xFFFFFFFF, step >> 32]
        assert oracle.group_noise_bits(seed, step, row, k) == int(oracle.philox4x32_10(key, ctr)[0])
    assert ((2**31 - 1) >> 2) < 0x40000000


def test_philox_words_are_uniform():
    # 2^18 words from consecutive ids of a few rows: top byte histogram is flat.
    f = oracle.lib().fso_noise_bits
    words = np.array([f(0, 3, row, v) for row in range(4) for v in range(1 << 16)], dtype=np.uint64)
    counts = np.bincount((words >> np.uint64(24)).astype(np.int64), minlength=256)
    exp = words.size / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    from scipy.stats import chi2 as chi2_dist
    assert chi2_dist.sf(chi2, 255) > 1e-4


# --- the uniform -> Gumbel transform --------------------------------------

getcontext().prec = 60
_TWO32P1 = Decimal(2**32 + 1)


def _gumbel_decimal(r: int) -> Decimal:
    u = Decimal(r + 1) / _TWO32P1
    return -((-(u.ln())).ln())


def test_gumbel_transform_against_decimal_arithmetic():
    rng = np.random.default_rng(3)
    rs = [0, 1, 2, 3, 2**31 - 2, 2**31 - 1, 2**31, 2**31 + 1, 2**32 - 3, 2**32 - 2, 2**32 - 1]
    rs += [int(x) for x in rng.integers(0, 2**32, 400, dtype=np.uint64)]
    rs += [2**32 - int(x) for x in rng.integers(1, 2**12, 100)]  # u close to 1: cancellation region
    for r in rs:
        ref = float(_gumbel_decimal(r))
        got = oracle.gumbel64(r)
        assert abs(got - ref) <= 4e-15 * max(1.0, abs(ref)), (r, got, ref)
        # the fp32 value the decision uses is the fp64 value rounded once
        assert oracle.gumbel32(r) == np.float32(ref) or abs(oracle.gumbel32(r) - ref) <= 1.2e-7 * max(1, abs(ref))


def test_gumbel_endpoints_closed_form():
    # u ranges over (r+1)/(2^32+1): the extremes are g(0) = -ln ln(2^32+1) and
    # g(2^32-1) = -ln ln(1 + 2^-32), both finite.
    g_min = -math.log(math.log(2.0**32 + 1.0))
    g_max = -math.log(math.log1p(2.0**-32))
    assert abs(oracle.gumbel64(0) - g_min) < 1e-14
    assert abs(oracle.gumbel64(2**32 - 1) - g_max) < 1e-13
    assert abs(g_min - (-3.0992230)) < 1e-6 and abs(g_max - 22.1807098) < 1e-6


def test_gumbel_cdf_counts_match_closed_form():
    # The transform is increasing in r, so #{r : g(r) <= x} is found by bisection.  With
    # u_r = (r+1)/(2^32+1), g(r) <= x iff r + 1 <= F(x) (2^32 + 1), F(x) = exp(-exp(-x)).
    def count_le(x):
        lo, hi = 0, 2**32  # count in [lo, hi]
        while lo < hi:
            mid = (lo + hi) // 2
            if oracle.gumbel64(mid) <= x:
                lo = mid + 1
            else:
                hi = mid
        return lo

    getcontext().prec = 60
    for x in [-2.5, -1.0, -0.3, 0.0, 0.5, 1.0, 2.0, 4.0, 8.0, 15.0]:
        F = (-(-Decimal(x)).exp()).exp()
        expect = int((F * _TWO32P1).to_integral_value(rounding="ROUND_FLOOR"))
        assert abs(count_le(x) - expect) <= 1, x


@pytest.mark.slow
def test_gumbel_exhaustive_all_words_finite_and_monotone():
    # Every one of the 2^32 words gives a finite fp32 noise value, non-decreasing in r.
    nonfinite, decreases, mn, mx = oracle.gumbel_scan(0, 2**32)
    assert nonfinite == 0
    assert decreases == 0
    assert mn == float(np.float32(-math.log(math.log(2.0**32 + 1.0))))
    assert mx == float(np.float32(-math.log(math.log1p(2.0**-32))))


def test_gumbel_moments():
    # Mean over a uniform grid of words ~ Euler-Mascheroni gamma, variance ~ pi^2 / 6.
    stride = 4096
    g = np.array([oracle.gumbel64(r) for r in range(stride // 2, 2**32, stride)])
    assert abs(g.mean() - 0.5772156649015329) < 2e-3
    assert abs(g.var() - math.pi**2 / 6) < 5e-3
