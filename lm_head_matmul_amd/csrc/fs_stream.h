// fs_stream.h -- the streaming FMMS kernels for MI355X (gfx950 / CDNA4).
//
// Fused LM-head matmul + sample (FMMS): logits are computed tile by tile on
// chip, Gumbel noise is added, each vocabulary tile keeps one (value, index)
// maximizer per row, and a small reduction over tiles yields the sample; the
// [B, V] logits never reach HBM.  Exact because argmax decomposes over a
// partition of the vocabulary.  [FlashSampling, arXiv 2603.15854, abstract;
// readus.org FlashSampling summary, section on the two-stage FMMS kernel]
//
// Layout on the device (one persistent workgroup per vocabulary tile, one tile
// per CU):
//  * A tile is a contiguous, balanced range of 16-row vocab blocks.  Waves
//    stream their blocks' rows of W straight from HBM into VGPRs in the MFMA
//    operand layout: lane (r, g) = (lane % 16, lane / 16) holds row r, and lane
//    group g the k values its 16-byte loads bring (the lane k-layout); H is
//    read with the same k permutation, so each MFMA still sums over 32
//    matching k values.
//  * H (the small operand) sits in LDS: the whole [B, d] when it fits,
//    otherwise k-chunks copied straight from global memory into LDS buffers
//    (LDS-direct loads) a chunk or two ahead of their use.  Rows are padded by
//    16 bytes so the B-operand reads of 16 lanes land in distinct banks.
//  * Up to 64 batch rows: 8 waves per workgroup (the round-major kernel with H
//    resident, the chunk-outer kernel otherwise); 65 .. 256 rows: the
//    register-blocked wide kernel, 4 waves.
//  * Epilogue, on the accumulators: scale by 1/T, mask, Philox4x32-10 noise
//    (one call covers the four consecutive vocab ids a lane holds), argmax
//    update (top-k: a short candidate list per lane instead).  Per tile, the
//    winners go to a [B, n_tiles] workspace, which a second small launch on the
//    same stream reduces over tiles.
#pragma once

#include <atomic>

#include "fs_device.h"
#include "fs_kernels.h"

namespace fsk {

// One butterfly step at lane distance OFF of the (value, index) maximizer and,
// grouped, of the log-sum-exp state: each lane merges its partner's (both
// merges are symmetric, so the pair ends equal).
template <int EPI, int OFF>
__device__ __forceinline__ void best_step(float& v, int32_t& i, float& m, float& s) {
  merge_best(v, i, lane_xor_f<OFF>(v), (int32_t)lane_xor<OFF>((uint32_t)i));
  if (EPI == EPI_GROUP) {
    const float om = lane_xor_f<OFF>(m), os = lane_xor_f<OFF>(s);
    lse_merge(m, s, om, os);
  }
}

// ---------------------------------------------------------------------------
// Cross-tile reduction: a second, small launch on the same stream (the kernel
// boundary publishes the workspace), one wave per batch row over its n_tiles
// entries.  [FlashSampling, arXiv 2603.15854, abstract: a small reduction over
// the per-tile maximizers finishes the sample]
// ---------------------------------------------------------------------------
// With several groups per launch (gridDim.y groups of tpg tiles each), group
// g reduces tiles [g * tpg, (g + 1) * tpg) into out_sum[g * out_stride + b].
template <int EPI>
__global__ void __launch_bounds__(kThreads)
    reduce_tiles_kernel(const int B, const int n_tiles, const float* __restrict__ ws_val,
                        const int32_t* __restrict__ ws_idx, const float* __restrict__ ws_m,
                        const float* __restrict__ ws_s, int32_t* __restrict__ out_idx,
                        GroupSummary* __restrict__ out_sum, const int tpg, const int64_t out_stride) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (b >= B) return;
  const int t0 = blockIdx.y * tpg;
  float v = -INFINITY, m = -INFINITY, s = 0.0f;
  int32_t i = -1;
  // A lane's tiles in batches of kPer, every load of a batch issued before any
  // merge: one memory round trip per batch (with a wait per tile, this launch
  // took ~5 us at 256 tiles).  Slots past the end merge the neutral entry.
  constexpr int kPer = 4;
  const int64_t row = (int64_t)b * n_tiles;
  for (int t1 = t0 + lane; t1 < t0 + tpg; t1 += 64 * kPer) {
    float vv[kPer], mm[kPer], ss[kPer];
    int32_t ii[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool ok = t1 + 64 * u < t0 + tpg;
      const int64_t o = row + (ok ? t1 + 64 * u : t1);
      const float lv = ws_val[o];
      const int32_t li = ws_idx[o];
      vv[u] = ok ? lv : -INFINITY;
      ii[u] = ok ? li : -1;
      if (EPI == EPI_GROUP) {
        const float lm = ws_m[o], ls = ws_s[o];
        mm[u] = ok ? lm : -INFINITY;
        ss[u] = ok ? ls : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      merge_best(v, i, vv[u], ii[u]);
      if (EPI == EPI_GROUP) lse_merge(m, s, mm[u], ss[u]);
    }
  }
  best_step<EPI, 32>(v, i, m, s);
  best_step<EPI, 16>(v, i, m, s);
  best_step<EPI, 8>(v, i, m, s);
  best_step<EPI, 4>(v, i, m, s);
  best_step<EPI, 2>(v, i, m, s);
  best_step<EPI, 1>(v, i, m, s);
  if (lane == 0) {
    if (EPI == EPI_GROUP) {
      GroupSummary g;
      g.lse = (m == -INFINITY) ? -INFINITY : m + logf(s);
      g.pmax = v;
      g.arg = i;
      out_sum[(int64_t)blockIdx.y * out_stride + b] = g;
    } else {
      out_idx[b] = i;
    }
  }
}

// Per-wave results (already reduced inside the wave) sit in LDS scratch as
// [kWaves][Bp] (val, idx, m, s); reduce over waves and publish the tile's entry.
template <int EPI, int WAVES = kWaves>
__device__ void publish_tile(const StreamParams& p, const int Bp, const float* sv, const int32_t* si, const float* sm,
                             const float* ss) {
  const int tile = blockIdx.x;
  for (int b = threadIdx.x; b < p.B; b += WAVES * 64) {
    float v = -INFINITY, m = -INFINITY, s = 0.0f;
    int32_t i = -1;
    for (int w = 0; w < WAVES; ++w) {
      merge_best(v, i, sv[w * Bp + b], si[w * Bp + b]);
      if (EPI == EPI_GROUP) lse_merge(m, s, sm[w * Bp + b], ss[w * Bp + b]);
    }
    const int64_t o = (int64_t)b * p.n_tiles + tile;
    p.ws_val[o] = v;
    p.ws_idx[o] = i;
    if (EPI == EPI_GROUP) {
      p.ws_m[o] = m;
      p.ws_s[o] = s;
    }
    if (p.dbg_max) {
      p.dbg_max[o] = v;
      p.dbg_arg[o] = i;
    }
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the streaming kernels.
// ---------------------------------------------------------------------------
struct TileRange {
  int64_t mb_lo, mb_hi;
  int rounds;
};

// Online grouped summaries: true once this tile's group has been published
// (ready[g] == ready_epoch, read with system-scope loads, so a flag in host
// memory or one written by another stream's work is seen), false if the wait
// ran out (then *status is set).  Thread 0 polls with relaxed loads, sleeping
// between reads, and acquires once (a fence after the load that saw the
// epoch): on this GPU an acquire invalidates the XCD's L2, which a poll loop of
// acquire loads would do on every read, under the tiles of published groups
// that are streaming beside it.  The barrier hands the answer, and the
// acquire's ordering, to the workgroup.
// [arXiv 2603.15854 abstract: grouped variants for online settings; readus.org
// FlashSampling summary, "Group Gumbel Max": the groups stream past, each one
// summarized as it comes]
__device__ __forceinline__ bool group_published(const StreamParams& p) {
  __shared__ int ok;
  if (threadIdx.x == 0) {
    const int g = (int)(blockIdx.x / (unsigned)p.group_tiles);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    int r = 0;
    for (;;) {
      if (__hip_atomic_load(p.ready + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == p.ready_epoch) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // system scope
        r = 1;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.wait_ticks) break;
      __builtin_amdgcn_s_sleep(8);
    }
    if (!r) __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    ok = r;
  }
  __syncthreads();
  return ok != 0;
}

__device__ __forceinline__ TileRange tile_range(const StreamParams& p) {
  TileRange t;
  if (p.group_tiles > 0) {  // balanced inside each group
    const int g = blockIdx.x / p.group_tiles, j = blockIdx.x - g * p.group_tiles;
    t.mb_lo = (int64_t)g * p.group_blocks + (int64_t)j * p.group_blocks / p.group_tiles;
    t.mb_hi = (int64_t)g * p.group_blocks + (int64_t)(j + 1) * p.group_blocks / p.group_tiles;
  } else {
    t.mb_lo = tile_lo(blockIdx.x, p.n_mblocks, p.n_tiles, p.tile_ratio);
    t.mb_hi = tile_lo(blockIdx.x + 1, p.n_mblocks, p.n_tiles, p.tile_ratio);
  }
  t.rounds = (int)((t.mb_hi - t.mb_lo + kWaves - 1) / kWaves);
  return t;
}

// H row, noise row and noise step of batch row b of a launch (see
// StreamParams::samples).
struct VRow {
  int h;
  uint32_t row, step_lo, step_hi;
};

__device__ __forceinline__ VRow vrow_of(const StreamParams& p, int b) {
  VRow v;
  v.step_lo = p.step_lo;
  v.step_hi = p.step_hi;
  if (p.samples <= 1) {
    v.h = b;
  } else {
    const int r = p.vrow0 + b;
    v.h = r / p.samples;
    const uint32_t smp = (uint32_t)(r - v.h * p.samples);
    v.step_lo = p.step_lo + smp;
    v.step_hi = p.step_hi + (v.step_lo < smp ? 1u : 0u);
  }
  v.row = (uint32_t)(p.row_offset + v.h);
  return v;
}

// H chunk `cidx` (k in [cidx*cs*256, ...)) as 16-byte pieces: piece P = n * (cs*32) + q.
// The load is unconditional (row and k clamped into H); h_valid says whether
// the piece lies inside H (pieces outside are stored as zero).
__device__ __forceinline__ u32x4_t h_load(const StreamParams& p, int cidx, int P) {
  const int per_row = p.cs * 32;
  const int n = P / per_row;
  const int q = P - n * per_row;
  const int k = cidx * p.cs * 256 + q * 8;
  const int nc = n < p.B ? n : p.B - 1;
  const int kc = k < p.d ? k : p.d - 8;
  return *(const u32x4_t*)(p.H + (int64_t)vrow_of(p, nc).h * p.ldh + kc);
}

__device__ __forceinline__ bool h_valid(const StreamParams& p, int cidx, int P) {
  const int per_row = p.cs * 32;
  const int n = P / per_row;
  const int k = cidx * p.cs * 256 + (P - n * per_row) * 8;
  return n < p.B && k < p.d;
}

__device__ __forceinline__ void h_store(const StreamParams& p, unsigned char* buf, int P, u32x4_t v) {
  const int per_row = p.cs * 32;
  const int n = P / per_row;
  const int q = P - n * per_row;
  *(u32x4_t*)(buf + n * p.h_rowstride + q * 16) = v;
}

// Stages the whole chunk at kernel start: rows >= B are zero-filled without
// loads; the valid rows go in batches of kMaxStagePieces loads per thread, so
// a thread waits once per batch rather than once per piece.
__device__ void h_stage_all(const StreamParams& p, int cidx, unsigned char* buf) {
  const int per_row = p.cs * 32;
  const int nv = p.B * per_row, np = p.h_rows * per_row;
  for (int P = nv + threadIdx.x; P < np; P += kThreads) h_store(p, buf, P, u32x4_t{0u, 0u, 0u, 0u});
  for (int P0 = 0; P0 < nv; P0 += kMaxStagePieces * kThreads) {
    u32x4_t v[kMaxStagePieces];
#pragma unroll
    for (int i = 0; i < kMaxStagePieces; ++i) {
      const int P = P0 + threadIdx.x + i * kThreads;
      v[i] = h_load(p, cidx, P < nv ? P : nv - 1);
    }
#pragma unroll
    for (int i = 0; i < kMaxStagePieces; ++i) {
      const int P = P0 + threadIdx.x + i * kThreads;
      if (P < nv) h_store(p, buf, P, h_valid(p, cidx, P) ? v[i] : u32x4_t{0u, 0u, 0u, 0u});
    }
  }
}

// Prefetch of the next chunk into registers: raw, unconditional loads (so the
// W stream in flight is never drained by a wait); masking happens at commit.
__device__ __forceinline__ void h_prefetch(u32x4_t (&hs)[kMaxStagePieces], const StreamParams& p, int cidx) {
  const int np = p.h_rows * p.cs * 32;
#pragma unroll
  for (int i = 0; i < kMaxStagePieces; ++i) {
    const int P = threadIdx.x + i * kThreads;
    hs[i] = h_load(p, cidx, P < np ? P : np - 1);
  }
}

__device__ __forceinline__ void h_commit(const u32x4_t (&hs)[kMaxStagePieces], const StreamParams& p, int cidx,
                                         unsigned char* buf) {
  const int np = p.h_rows * p.cs * 32;
#pragma unroll
  for (int i = 0; i < kMaxStagePieces; ++i) {
    const int P = threadIdx.x + i * kThreads;
    if (P < np) h_store(p, buf, P, h_valid(p, cidx, P) ? hs[i] : u32x4_t{0u, 0u, 0u, 0u});
  }
}

// One LDS-direct copy of 16 bytes per lane: the wave's 64 lanes fill the 1 KB
// from lds (lane i at lds + 16 i).  It is written in inline assembly so that
// the compiler leaves it out of its count of loads in flight.  With the
// builtin, the next use of any load issued before a copy waited for every load
// in flight (vmcnt 0), which drained the W prefetch once per H chunk.  The
// compiler's own waits for W stay correct: a copy it does not count can only
// make them wait longer.  The kernels order the copies themselves by explicit
// waits before the barrier that hands a chunk to its readers.
// m0 (the LDS address) is reserved to the compiler, which does not track this
// write to it.  That is safe only while no compiler-generated instruction in
// these kernels uses m0; a CPU test checks that on the generated assembly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* src, unsigned char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
// The same copy from a wave-uniform base plus a 32-bit lane byte offset.
__device__ __forceinline__ void lds_copy16_s(const void* base, uint32_t off, unsigned char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Stage H chunk `cidx` (two 256-wide sub-blocks: 1 KB per row) straight from
// global memory into LDS, without registers: one wave instruction moves one row
// (lane l carries bytes [16 l, 16 l + 16) of it).  Rows b < B (wave
// b % kWaves issues row b); the zero row is written once at kernel start.  The
// loads retire in order with the W loads of the issuing wave.  The copies are
// a fixed, fully unrolled sequence of ROWS rows per wave (row b of wave w is
// w + 8k) with no branches: rows past B repeat row B - 1, which writes the
// same bytes to the same place.
template <int ROWS>
__device__ __forceinline__ void h_chunk_dma(const StreamParams& p, int cidx, unsigned char* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* src = p.H + cidx * 512 + lane * 8;
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    const int b0 = wave + k * kWaves;
    const int b = b0 < p.B ? b0 : p.B - 1;
    lds_copy16(src + (int64_t)vrow_of(p, b).h * p.ldh, buf + b * p.h_rowstride);
  }
}

// The vocabulary mask of the tile, staged in LDS at kernel start: rows b < B,
// words [w_lo, w_lo + p.mask_words) of each row (the host sizes batch chunks so
// that it always fits).  Reading mask bits from LDS keeps global loads out of
// the epilogue: the vector-memory counter is in order, so waiting for one mask
// word would also wait for every W prefetch issued before it.
__device__ __forceinline__ int64_t mask_w_lo(const StreamParams& p, const TileRange& tr) {
  return (p.vocab_offset + tr.mb_lo * 16) >> 5;
}

__device__ void mask_stage(const StreamParams& p, const TileRange& tr, uint32_t* lds) {
  if (!p.mask) return;
  const int64_t w_lo = mask_w_lo(p, tr);
  const int64_t w_max = (p.vocab_offset + p.V - 1) >> 5;  // last word of the launch's vocabulary
  const int n = p.B * p.mask_words;
  for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
    uint32_t w4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + threadIdx.x + j * kThreads;
      const int ii = i < n ? i : n - 1;
      const int b = ii / p.mask_words;
      int64_t w = w_lo + (ii - b * p.mask_words);
      w = w <= w_max ? w : w_max;
      w4[j] = p.mask[(int64_t)vrow_of(p, b).row * p.ldm + w];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + threadIdx.x + j * kThreads;
      if (i < n) {
        const int b = i / p.mask_words;
        lds[i] = (w_lo + (i - b * p.mask_words) <= w_max) ? w4[j] : 0u;
      }
    }
  }
}

// Four mask bits of vocab ids gv0 .. gv0+3 (gv0 % 4 == 0) of local row b.
// Kernels without a mask are compiled with MASKED = false: no mask code at all.
template <bool MASKED>
__device__ __forceinline__ uint32_t mask_bits4(const StreamParams& p, const uint32_t* lds, int64_t w_lo, int64_t gv0,
                                               int b) {
  if (!MASKED) return 0xFu;
  const uint32_t word = lds[b * p.mask_words + (int)((gv0 >> 5) - w_lo)];
  return (word >> (uint32_t)(gv0 & 31)) & 0xFu;
}

// Perturbed scores of the four consecutive vocab ids v0 .. v0+3 (local ids,
// v0 % 4 == 0) of row b, given their raw logits and mask bits; updates the
// running maximizer (and the log-sum-exp state in grouped mode).  The scan
// order of a lane is increasing in v, so a strict comparison keeps the lowest
// id on ties.
// Gumbel noise of the four consecutive vocab ids gv0 .. gv0+3 (gv0 % 4 == 0,
// global ids) of batch row b of the launch: one Philox call.  MULTI = false
// for kernels that only run launches of one sample per row (the row is then
// row_offset + b, with no division).
template <bool MULTI = true>
__device__ __forceinline__ f32x4_t noise_quad(const StreamParams& p, int gv0, int b) {
  const VRow v = MULTI ? vrow_of(p, b) : VRow{b, (uint32_t)(p.row_offset + b), p.step_lo, p.step_hi};
  const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)gv0 >> 2, v.row, v.step_lo, v.step_hi);
  return f32x4_t{gumbel_from_bits(r.w[0]), gumbel_from_bits(r.w[1]), gumbel_from_bits(r.w[2]),
                 gumbel_from_bits(r.w[3])};
}

// The tile's noise table in LDS (when planned, p.noise_pitch > 0): rows b < B,
// one float per vocab id of the tile, written by all threads before the stream
// starts (made visible by the driver's first barrier).
__device__ void noise_stage(const StreamParams& p, const TileRange& tr, float* lds) {
  const int quads = (int)(tr.mb_hi - tr.mb_lo) * 4;
  const int n = p.B * quads;
  const int v_base = (int)p.vocab_offset + (int)(tr.mb_lo * 16);
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int b = i / quads;
    const int q = i - b * quads;
    *(f32x4_t*)(lds + b * p.noise_pitch + q * 4) = noise_quad(p, v_base + q * 4, b);
  }
}

// Perturbed scores of the four consecutive vocab ids v0 .. v0+3 (local ids,
// v0 % 4 == 0) given their raw logits, noise and mask bits; updates the
// running maximizer (and the log-sum-exp state in grouped mode).  The scan
// order of a lane is increasing in v, so a strict comparison keeps the lowest
// id on ties.  Vocabulary ids are below 2^31 (checked by the API), so the
// epilogue works in 32-bit integers.
template <int EPI>
__device__ __forceinline__ void epilogue_quad(const StreamParams& p, int v0, const float (&acc)[4], const f32x4_t g,
                                              uint32_t bits, float& bv, int32_t& bi, float& lm, float& ls) {
  const int gv0 = (int)p.vocab_offset + v0;
  const int rem = (int)p.V - v0;
  const uint32_t ok4 = bits & (rem >= 4 ? 0xFu : (rem <= 0 ? 0u : (1u << rem) - 1u));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = (ok4 >> i) & 1u;
    const float s = acc[i] * p.inv_t;
    const float pv = ok ? s + g[i] : -INFINITY;
    if (pv > bv) {
      bv = pv;
      bi = gv0 + i;
    }
    if (EPI == EPI_GROUP && ok) lse_push(lm, ls, s);
  }
}

// ---------------------------------------------------------------------------
// Fused top-k epilogue.  [readus.org FlashSampling summary, section on Top-K
// and masking: a pre-filter keeps a candidate set, then exact Gumbel-Max runs
// inside it]  The exact top-k of a row is contained in the union of every
// part's own top-k, for any partition of the vocabulary; a part that keeps
// fewer entries is still exact as long as everything it dropped ranks below
// the row's k-th kept score.  So each lane keeps its kTopkLane best (score,
// id) pairs and counts what it saw; the workgroup merges its lanes' lists
// per batch row into kTopkLane entries plus a bound on every dropped key,
// which the merge kernel checks against the row's k-th key (and recomputes the
// tile's ids where the check fails).
// ---------------------------------------------------------------------------
struct TopkList {
  float s[kTopkLane];  // descending; -inf marks an empty entry
  int32_t id[kTopkLane];
  int seen;  // ids pushed: more than kTopkLane means some were dropped
};

__device__ __forceinline__ void topk_init(TopkList& t) {
#pragma unroll
  for (int j = 0; j < kTopkLane; ++j) {
    t.s[j] = -INFINITY;
    t.id[j] = -1;
  }
  t.seen = 0;
}

// Inserts (s, id).  A lane meets its ids in increasing order, so a strict
// comparison keeps the lower id of two equal scores first, and anything it
// drops ranks below its last entry.  NaN never enters (and counts as seen).
__device__ __forceinline__ void topk_push(TopkList& t, float s, int32_t id) {
  static_assert(kTopkLane == 4, "the insertion below is written for four entries");
  const bool c0 = s > t.s[0], c1 = s > t.s[1], c2 = s > t.s[2], c3 = s > t.s[3];
  ++t.seen;
  t.s[3] = c2 ? t.s[2] : (c3 ? s : t.s[3]);
  t.id[3] = c2 ? t.id[2] : (c3 ? id : t.id[3]);
  t.s[2] = c1 ? t.s[1] : (c2 ? s : t.s[2]);
  t.id[2] = c1 ? t.id[1] : (c2 ? id : t.id[2]);
  t.s[1] = c0 ? t.s[0] : (c1 ? s : t.s[1]);
  t.id[1] = c0 ? t.id[0] : (c1 ? id : t.id[1]);
  t.s[0] = c0 ? s : t.s[0];
  t.id[0] = c0 ? id : t.id[0];
}

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t u64_min(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Two sorted lists of four keys (k: this lane's, the partner lane's at lane
// distance OFF) and bounds h on what each dropped: afterwards k is the best
// four of both, descending, and h bounds everything dropped (the larger bound
// and the best key of the four not kept).  One step of a bitonic merge: the
// elementwise maxima of one list and the other reversed are the best four, the
// minima the four dropped.
template <int OFF>
__device__ __forceinline__ void topk_merge_lists(uint64_t (&k)[kTopkLane], uint64_t& h) {
  static_assert(kTopkLane == 4, "the merge below is written for four entries");
  uint64_t q[kTopkLane];
#pragma unroll
  for (int j = 0; j < kTopkLane; ++j) q[j] = lane_xor64<OFF>(k[j]);
  h = u64_max(h, lane_xor64<OFF>(h));
  uint64_t top[kTopkLane];
#pragma unroll
  for (int j = 0; j < kTopkLane; ++j) {
    top[j] = u64_max(k[j], q[kTopkLane - 1 - j]);
    h = u64_max(h, u64_min(k[j], q[kTopkLane - 1 - j]));
  }
  // top is bitonic: two compare-exchange stages sort it descending
  const uint64_t a0 = u64_max(top[0], top[2]), a2 = u64_min(top[0], top[2]);
  const uint64_t a1 = u64_max(top[1], top[3]), a3 = u64_min(top[1], top[3]);
  k[0] = u64_max(a0, a1);
  k[1] = u64_min(a0, a1);
  k[2] = u64_max(a2, a3);
  k[3] = u64_min(a2, a3);
}

// End of a top-k streaming kernel: per batch column, each wave merges its four
// lane groups' lists (lanes l16, l16 + 16, l16 + 32, l16 + 48); the waves'
// lists meet in LDS, where eight lanes per column merge the workgroup's eight
// into the tile's kTopkLane best keys and its bound -- the largest key it may
// have dropped (0 if none) -- which one lane writes to the candidate buffer.
// One list per tile keeps the buffer (and the merge launch's reads) an eighth
// of per-wave lists, and the write of a column's five words is one request per
// word instead of one per wave and word.
template <int NB>
__device__ __forceinline__ void finish_wave_topk(const StreamParams& p, unsigned char* smem, TopkList (&tk)[NB]) {
  constexpr int Bp = NB * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  __syncthreads();  // H buffers are free: reuse LDS as scratch
  uint64_t* sl = (uint64_t*)smem;  // [wave][column][kTopkSlot]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint64_t k[kTopkLane];
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j) k[j] = tk[nb].id[j] >= 0 ? topk_key(tk[nb].s[j], tk[nb].id[j]) : 0ull;
    // whatever the lane dropped ranks below its last entry (keys are distinct)
    uint64_t h = tk[nb].seen > kTopkLane && k[kTopkLane - 1] != 0 ? k[kTopkLane - 1] - 1 : 0ull;
    topk_merge_lists<16>(k, h);
    topk_merge_lists<32>(k, h);
    if (grp == 0) {
      uint64_t* d = sl + (wave * Bp + nb * 16 + l16) * kTopkSlot;
#pragma unroll
      for (int j = 0; j < kTopkLane; ++j) d[j] = k[j];
      d[kTopkLane] = h;
    }
  }
  __syncthreads();
  // thread t: column t / 8, wave t % 8's list (eight consecutive lanes of a wave)
  static_assert(kWaves == 8 && kThreads >= 8 * 64, "eight lists per column, 64 columns at most");
  const int b = (int)threadIdx.x >> 3, w = (int)threadIdx.x & 7;
  if (b < Bp) {  // uniform per wave: Bp is a multiple of 16
    const uint64_t* s = sl + (w * Bp + b) * kTopkSlot;
    uint64_t k[kTopkLane];
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j) k[j] = s[j];
    uint64_t h = s[kTopkLane];
    topk_merge_lists<1>(k, h);
    topk_merge_lists<2>(k, h);
    topk_merge_lists<4>(k, h);
    if (w == 0 && b < p.B) {
      uint64_t* dst = p.topk_cand + (int64_t)b * kTopkSlot * p.n_tiles + blockIdx.x;
#pragma unroll
      for (int j = 0; j < kTopkLane; ++j) dst[(int64_t)j * p.n_tiles] = k[j];
      dst[(int64_t)kTopkLane * p.n_tiles] = h;
    }
  }
}

// Top-k epilogue of four consecutive ids v0 .. v0+3 (local ids) of one batch
// row: the allowed, in-range ones enter the lane's list.
__device__ __forceinline__ void topk_quad(const StreamParams& p, int v0, const float (&acc)[4], uint32_t bits,
                                          TopkList& t) {
  const int gv0 = (int)p.vocab_offset + v0;
  const int rem = (int)p.V - v0;
  const uint32_t ok4 = bits & (rem >= 4 ? 0xFu : (rem <= 0 ? 0u : (1u << rem) - 1u));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((ok4 >> i) & 1u) topk_push(t, acc[i] * p.inv_t, gv0 + i);
}

// Lane's W row pointer for vocab block `mb` (rows past the tile or past V are
// clamped to the tile's last row; their results are never used).
__device__ __forceinline__ const uint16_t* w_row(const StreamParams& p, const TileRange& tr, int64_t mb, int l16) {
  const int64_t tile_end = (tr.mb_hi * 16 < p.V ? tr.mb_hi * 16 : p.V);
  int64_t row = mb * 16 + l16;
  row = row < tile_end ? row : tile_end - 1;
  return p.W + row * p.ldw;
}

template <int LAYOUT>
__device__ __forceinline__ int lane_base(int g) {
  return LAYOUT == 0 ? g * 128 : LAYOUT == 1 ? g * 16 : (g >> 1) * 256 + (g & 1) * 16;
}
template <int LAYOUT>
constexpr int lane_step() {
  return LAYOUT == 0 ? 16 : LAYOUT == 1 ? 64 : 32;
}

// W addressing of the streaming loops: a scalar base per 16-row block plus a
// 32-bit lane offset (row l16 and the lane group's 128 bytes).  Both lane
// offsets are computed once: rows of the tile's last block are clamped to the
// tile's last row (a partial block at the end of the vocabulary).  Keeping the
// multiply out of the loop matters: the fused 32-bit multiply-add the compiler
// would otherwise emit per load writes a carry to scalar registers, which
// stalled the W stream on gfx950.
struct WLane {
  uint32_t full, last;
};

template <int LAYOUT>
__device__ __forceinline__ WLane w_lane(const StreamParams& p, const TileRange& tr, int l16, int grp) {
  const int64_t tile_end = tr.mb_hi * 16 < p.V ? tr.mb_hi * 16 : p.V;
  const int lim = (int)(tile_end - (tr.mb_hi - 1) * 16);  // rows of the last block, 1 .. 16
  const uint32_t ldw2 = (uint32_t)p.ldw * 2u;
  WLane w;
  w.full = (uint32_t)l16 * ldw2 + (uint32_t)lane_base<LAYOUT>(grp);
  w.last = (uint32_t)(l16 < lim ? l16 : lim - 1) * ldw2 + (uint32_t)lane_base<LAYOUT>(grp);
  return w;
}

// The 8 x 16 bytes lane (l16, grp) owns of 256-wide sub-block sb of 16-row
// block mb (uniform across the wave).  A block past the tile (a wave idle in
// the tile's last round) reads the tile's last block; its results are
// discarded.
template <int LAYOUT>
__device__ __forceinline__ void w_load8(const StreamParams& p, const TileRange& tr, const WLane& wl, int64_t mb,
                                        int sb, u32x4_t (&buf)[8]) {
  mb = mb < tr.mb_hi ? mb : tr.mb_hi - 1;
  const char* base = (const char*)(p.W + mb * 16 * p.ldw) + sb * 512;
  const uint32_t off = mb == tr.mb_hi - 1 ? wl.last : wl.full;
#pragma unroll
  for (int e = 0; e < 8; ++e) buf[e] = *(const u32x4_t*)(base + off + e * lane_step<LAYOUT>());
}

// ---------------------------------------------------------------------------
// Streaming drivers.  Both call
//   body(cur, hbase, sbc, r, t)  -- consume sub-block t (0 .. nsub-1) of round r;
//                                   hbase/sbc locate its H slice in LDS
//   round_end(r)                 -- after the last sub-block of round r
// Wave w of the workgroup owns vocab block mb_lo + r * 8 + w in round r.
//
// Fast driver (d % (256 U) == 0; chunked H only with chunks of exactly U
// sub-blocks): rounds are split into groups of U sub-blocks whose bodies run
// unconditionally, with a ring of U register buffers: while sub-block t is
// consumed the loads of t + 1 .. t + U - 1 are in flight (they run on into the
// next round).  The loop body has no data-dependent branches, so the
// compiler's wait counters stay exact and no prefetch is ever drained.
// ---------------------------------------------------------------------------
template <int U, bool RESIDENT, int LAYOUT, class Body, class RoundEnd, class Pre>
__device__ __forceinline__ void stream_driver_fast(const StreamParams& p, const TileRange& tr, unsigned char* smem,
                                                   Body&& body, RoundEnd&& round_end, Pre&& pre) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int nsub = p.nsub, ngrp = nsub / U;
  const int bufbytes = p.h_rows * p.h_rowstride;
  if (tr.rounds == 0) return;

  // per-lane 64-bit row addresses: measured faster here than a scalar block
  // base plus a lane offset (w_load8), unlike in the chunk-outer kernel
  auto load = [&](u32x4_t (&buf)[8], int r, int sb) {
    const char* src = (const char*)(w_row(p, tr, tr.mb_lo + (int64_t)r * kWaves + wave, l16) + sb * 256) +
                      lane_base<LAYOUT>(grp);
#pragma unroll
    for (int e = 0; e < 8; ++e) buf[e] = *(const u32x4_t*)(src + e * lane_step<LAYOUT>());
  };
  int lr = 0, lsb = 0;  // next position to load; stays on the last sub-block past the end
  auto advance = [&]() {
    if (++lsb == nsub) {
      lsb = 0;
      ++lr;
    }
    if (lr >= tr.rounds) {
      lr = tr.rounds - 1;
      lsb = nsub - 1;
    }
  };

  // The first W items go out before anything else: their latency overlaps the
  // kernel's own staging (pre: mask words, noise table) and H's.
  u32x4_t buf[U][8];
#pragma unroll
  for (int k = 0; k < U - 1; ++k) {
    load(buf[k], lr, lsb);
    advance();
  }
  pre();

  // Chunked H (chunks of U = 2 sub-blocks, 1 KB per row): chunks are copied
  // straight into LDS (h_chunk_dma), the zero row of both buffers once here.
  static_assert(RESIDENT || U == 2, "chunked H in the fast driver: two sub-blocks per chunk");
  if (RESIDENT) {
    h_stage_all(p, 0, smem);
  } else {
    for (int i = threadIdx.x; i < (p.h_rows - p.B) * 64; i += kThreads) {
      const int row = p.B + i / 64, q = i % 64;
      *(u32x4_t*)(smem + row * p.h_rowstride + q * 16) = u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t*)(smem + bufbytes + row * p.h_rowstride + q * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
    h_chunk_dma<kMfmaMaxB / kWaves>(p, 0, smem);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS copies have landed
  }
  __syncthreads();

  int cc = 0;  // chunks consumed (chunked H: one chunk per group)
  for (int r = 0; r < tr.rounds; ++r) {
    for (int g = 0; g < ngrp; ++g) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        load(buf[(k + U - 1) % U], lr, lsb);
        advance();
        // the chunk after this one (chunk index == group index) into the other
        // buffer; past the last group of the last round this copies chunk 0
        // once more, unused
        if (!RESIDENT && k == 0)
          h_chunk_dma<kMfmaMaxB / kWaves>(p, g + 1 < ngrp ? g + 1 : 0, smem + ((cc + 1) & 1) * bufbytes);
        // keep the loads above ahead of the compute below: the scheduler would
        // otherwise sink them under the MFMAs to save registers
        __builtin_amdgcn_sched_barrier(0);
        if (RESIDENT)
          body(buf[k], smem, g * U + k, r, g * U + k);
        else
          body(buf[k], smem + (cc & 1) * bufbytes, k, r, g * U + k);
        if (!RESIDENT && k == U - 1) {
          // the copies were issued before the last W sub-block's 8 loads: once
          // at most those remain outstanding (vmcnt 8), this wave's copies landed
          __builtin_amdgcn_s_waitcnt(0xF78);
          __syncthreads();
          ++cc;
        }
      }
    }
    round_end(r);
  }
}

// Resident-H driver with blocks handed out on demand.  With H resident the
// waves of a workgroup share nothing while they stream but H, the tile's noise
// table and its mask words, so the tile's blocks need not be dealt in fixed
// rounds: wave w starts on block mb_lo + w, and each further block comes from
// a counter in LDS, taken as the wave starts its current block so that the
// prefetch of the next block's first sub-block knows where to read.  (With a
// fixed share per wave the second wave of each SIMD streamed at about half the
// rate of the first on MI355X, and the last ~45% of a workgroup's time ran on
// half of its waves.)
// body(buf, hbase, sbc, pblk, t): compute sub-block sbc of the current block,
// pblk being the wave's previous block (-1 before its second) whose epilogue
// may be finished at step t; block_end(cblk, pblk): the current block's
// accumulators are complete.  Returns the wave's last block, -1 if it had none.
template <int U, int LAYOUT, class Body, class BlockEnd, class Pre>
__device__ __forceinline__ int64_t stream_driver_dynamic(const StreamParams& p, const TileRange& tr,
                                                         unsigned char* smem, int* next_blk, Body&& body,
                                                         BlockEnd&& block_end, Pre&& pre) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int nsub = p.nsub, ngrp = nsub / U;
  if (tr.rounds == 0) return -1;  // an empty tile (the whole workgroup)
  auto load = [&](u32x4_t (&buf)[8], int64_t mb, int sb) {
    const char* src = (const char*)(w_row(p, tr, mb, l16) + sb * 256) + lane_base<LAYOUT>(grp);
#pragma unroll
    for (int e = 0; e < 8; ++e) buf[e] = *(const u32x4_t*)(src + e * lane_step<LAYOUT>());
  };
  int64_t cur = tr.mb_lo + wave;  // the wave's current block
  const bool any = cur < tr.mb_hi;
  if (!any) cur = tr.mb_hi - 1;  // loads of a wave without blocks stay in the tile; none is used
  int64_t nxt = -1;               // the block after the current one, -1 if none
  int64_t lb = cur;               // next position to load
  int lsb = 0;                    // position within the block
  // The kernel with noise in its epilogue takes each block's sub-blocks in an
  // order rotated per workgroup when rows have at most 8 of them (measured on
  // MI355X: small decode B=32 118.7 -> 110.6 us; at 16 sub-blocks, and in the
  // noise-table kernel, the rotation was slower).
  const int rot = (LAYOUT == kLayoutEpilogue && nsub <= 8) ? (int)(blockIdx.x % (unsigned)nsub) : 0;
  auto sb_at = [&](int j) { return j + rot < nsub ? j + rot : j + rot - nsub; };
  auto advance = [&]() {
    if (++lsb == nsub) {
      if (nxt >= 0) {
        lb = nxt;
        lsb = 0;
      } else {
        lsb = nsub - 1;  // past the wave's last block: stay on its last sub-block
      }
    }
  };

  // the first W items go out before the kernel's own staging (pre) and H's
  u32x4_t buf[U][8];
#pragma unroll
  for (int k = 0; k < U - 1; ++k) {
    load(buf[k], lb, sb_at(lsb));
    advance();
  }
  pre();
  h_stage_all(p, 0, smem);
  if (threadIdx.x == 0) *next_blk = (int)(tr.mb_lo + kWaves);
  __syncthreads();
  if (!any) return -1;

  int64_t pblk = -1;
  for (;;) {
    int got = 0;
    if (lane == 0) got = atomicAdd(next_blk, 1);
    got = __builtin_amdgcn_readfirstlane(got);
    nxt = got < tr.mb_hi ? got : -1;
    for (int g = 0; g < ngrp; ++g) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        load(buf[(k + U - 1) % U], lb, sb_at(lsb));
        advance();
        // keep the loads above ahead of the compute below
        __builtin_amdgcn_sched_barrier(0);
        body(buf[k], smem, sb_at(g * U + k), pblk, g * U + k);
      }
    }
    block_end(cur, pblk);
    pblk = cur;
    if (nxt < 0) break;
    cur = nxt;
  }
  return cur;
}

// General driver: any d (k tail clamped into the row's last chunk, which meets
// zeros in the staged H), any chunking, two register buffers.  Conditions are
// evaluated per sub-block.
template <bool RESIDENT, int LAYOUT, class Body, class RoundEnd, class Pre>
__device__ __forceinline__ void stream_driver_general(const StreamParams& p, const TileRange& tr, unsigned char* smem,
                                                      Body&& body, RoundEnd&& round_end, Pre&& pre) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int nsub = p.nsub, d = p.d;
  const int cs = RESIDENT ? nsub : p.cs;
  const int nchunk = RESIDENT ? 1 : p.nchunk;
  const int bufbytes = p.h_rows * p.h_rowstride;
  if (tr.rounds == 0) return;
  pre();

  auto load = [&](u32x4_t (&buf)[8], int r, int sb) {
    const uint16_t* base = w_row(p, tr, tr.mb_lo + (int64_t)r * kWaves + wave, l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = sb * 256 + (lane_base<LAYOUT>(grp) + e * lane_step<LAYOUT>()) / 2;
      buf[e] = *(const u32x4_t*)(base + (k < d ? k : d - 8));
    }
  };

  u32x4_t hs[kMaxStagePieces];
  if (RESIDENT) {
    h_stage_all(p, 0, smem);
  } else {
    h_prefetch(hs, p, 0);
    h_commit(hs, p, 0, smem);
  }
  __syncthreads();

  u32x4_t w0[8], w1[8];
  int r = 0, sb = 0, cidx = 0, sbc = 0, cc = 0;
  int lr = 0, lsb = 0;
  auto advance = [&]() {
    if (++lsb == nsub) {
      lsb = 0;
      ++lr;
    }
    if (lr >= tr.rounds) {
      lr = tr.rounds - 1;
      lsb = nsub - 1;
    }
  };
  load(w0, lr, lsb);
  advance();

  auto step = [&](const u32x4_t (&cur)[8], u32x4_t (&nxt)[8]) {
    load(nxt, lr, lsb);
    advance();
    __builtin_amdgcn_sched_barrier(0);
    if (RESIDENT) {
      body(cur, smem, sb, r, sb);
    } else {
      const bool chunk_end = (sbc == cs - 1 || sb == nsub - 1);
      const bool last_chunk = (r == tr.rounds - 1) && (cidx == nchunk - 1);
      const int next_c = cidx + 1 < nchunk ? cidx + 1 : 0;
      if (sbc == 0 && !last_chunk) h_prefetch(hs, p, next_c);
      body(cur, smem + ((p.nbuf == 2) ? (cc & 1) : 0) * bufbytes, sbc, r, sb);
      if (chunk_end) {
        if (!last_chunk) {
          if (p.nbuf == 2) {
            h_commit(hs, p, next_c, smem + ((cc + 1) & 1) * bufbytes);
            __syncthreads();
          } else {
            __syncthreads();
            h_commit(hs, p, next_c, smem);
            __syncthreads();
          }
        }
        ++cc;
        ++cidx;
        sbc = 0;
      } else {
        ++sbc;
      }
      if (sb == nsub - 1) {
        cidx = 0;
        sbc = 0;
      }
    }
    if (sb == nsub - 1) round_end(r);
    if (++sb == nsub) {
      sb = 0;
      ++r;
    }
  };

  const int total = tr.rounds * nsub;
  for (int it = 0; it < total; it += 2) {
    step(w0, w1);
    if (it + 1 < total) step(w1, w0);
  }
}

template <bool FAST, bool RESIDENT, int RING, int LAYOUT, class Body, class RoundEnd, class Pre>
__device__ __forceinline__ void stream_driver(const StreamParams& p, const TileRange& tr, unsigned char* smem,
                                              Body&& body, RoundEnd&& round_end, Pre&& pre) {
  if (FAST)
    stream_driver_fast<RING, RESIDENT, LAYOUT>(p, tr, smem, body, round_end, pre);
  else
    stream_driver_general<RESIDENT, LAYOUT>(p, tr, smem, body, round_end, pre);
}

// End of an MFMA streaming kernel: reduce each wave's maximizers over its four
// lane groups (lanes l16, l16 + 16, l16 + 32, l16 + 48 share a batch column),
// then over the waves through LDS, and publish the tile's entry.
template <int EPI, int NB, int WAVES = kWaves>
__device__ __forceinline__ void finish_wave_tile(const StreamParams& p, unsigned char* smem, float (&bv)[NB],
                                                 int32_t (&bi)[NB], float (&lm)[NB], float (&ls)[NB]) {
  constexpr int Bp = NB * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    best_step<EPI, 16>(bv[nb], bi[nb], lm[nb], ls[nb]);
    best_step<EPI, 32>(bv[nb], bi[nb], lm[nb], ls[nb]);
  }
  __syncthreads();  // H buffers are free: reuse LDS as scratch
  float* sv = (float*)smem;
  int32_t* si = (int32_t*)(sv + WAVES * Bp);
  float* sm = (float*)(si + WAVES * Bp);
  float* ss = sm + WAVES * Bp;
  if (grp == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + l16;
      sv[wave * Bp + b] = bv[nb];
      si[wave * Bp + b] = bi[nb];
      if (EPI == EPI_GROUP) {
        sm[wave * Bp + b] = lm[nb];
        ss[wave * Bp + b] = ls[nb];
      }
    }
  }
  __syncthreads();
  publish_tile<EPI, WAVES>(p, Bp, sv, si, sm, ss);
}

// ---------------------------------------------------------------------------
// MFMA streaming kernel (batch padded to 16 * NB columns).
//
// Deferred epilogue (NB <= 2): at the end of round r the accumulators move to
// a pending set, and N-block n of that set is finished (scale, mask, noise,
// argmax) in body n of round r + 1, right after that body's MFMAs; the last
// round is finished after the stream.  The ALU work of the epilogue is thereby
// spread over bodies whose W loads are already in flight.
// ---------------------------------------------------------------------------
// NOISE_LDS: the epilogue reads the tile's noise table staged in LDS before
// the stream (noise_stage); otherwise it runs Philox itself.  The two are
// separate kernels on purpose: with the Philox code inside the streaming loop
// the W stream ran about 9% slower on gfx950 even on rounds that took the
// table path, so the table kernels carry no Philox code in the loop at all.
template <int NB, int EPI, bool RESIDENT, bool FAST, bool MASKED, bool NOISE_LDS,
          int RING = (RESIDENT ? kFastRingResident : kFastRingChunked)>
__global__ void __launch_bounds__(kThreads) fmms_mfma_kernel(const StreamParams p) {
  constexpr int LAYOUT = EPI == EPI_STORE  ? kLayoutStore
                         : EPI == EPI_TOPK ? kLayoutTopk
                         : NOISE_LDS       ? kLayoutTable
                                           : kLayoutEpilogue;
  if constexpr (EPI == EPI_GROUP) {
    // the answer is the same in every lane; readfirstlane tells the compiler so
    if (p.ready && !__builtin_amdgcn_readfirstlane((int)group_published(p))) return;
  }
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range(p);
  const int rs = p.h_rowstride;
  uint32_t* mask_lds = (uint32_t*)(smem + p.mask_lds_off);
  const int64_t mw_lo = mask_w_lo(p, tr);
  const float* noise_lds = (const float*)(smem + p.noise_lds_off);
  // staged by the driver once the first W loads are out, visible after its first barrier
  auto pre = [&]() {
    if (MASKED) mask_stage(p, tr, mask_lds);
    if (EPI != EPI_STORE && NOISE_LDS) noise_stage(p, tr, (float*)noise_lds);
  };
  // H row of this lane in each 16-wide batch block (padding lanes read the zero row)
  int hoff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = nb * 16 + l16;
    hoff[nb] = lane_base<LAYOUT>(grp) + (row < p.B ? row : p.h_rows - 1) * rs;
  }

  float bv[NB], lm[NB], ls[NB];
  int32_t bi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = -INFINITY;
    bi[nb] = -1;
    lm[nb] = -INFINITY;
    ls[nb] = 0.0f;
  }
  f32x4_t acc[NB], pend[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    pend[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  TopkList tk[NB];  // EPI_TOPK only
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) topk_init(tk[nb]);

  // One sub-block: 8 k-steps; the B operands of step j + 1 are read from LDS
  // while the MFMAs of step j run.  (Left to itself the compiler waits on each
  // LDS read right before its MFMA, and the loop becomes bound by LDS latency.)
  auto compute = [&](const u32x4_t (&cur)[8], const unsigned char* hbase, int sbc) {
    const unsigned char* hb = hbase + sbc * 512;
    u32x4_t h0[NB], h1[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) h0[nb] = *(const u32x4_t*)(hb + hoff[nb]);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) h1[nb] = *(const u32x4_t*)(hb + hoff[nb] + (j + 1) * lane_step<LAYOUT>());
      __builtin_amdgcn_sched_barrier(0);  // reads of step j + 1 stay ahead of the MFMAs of step j
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[j]),
                                                          __builtin_bit_cast(bf16x8_t, h0[nb]), acc[nb], 0, 0, 0);
      if (j + 2 < 8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) h0[nb] = *(const u32x4_t*)(hb + hoff[nb] + (j + 2) * lane_step<LAYOUT>());
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[j + 1]),
                                                          __builtin_bit_cast(bf16x8_t, h1[nb]), acc[nb], 0, 0, 0);
    }
  };

  // Finish N-block nb of the pending accumulators of block mbg.
  auto finish_nb = [&](int64_t mbg, int nb) {
    if (mbg < 0 || mbg >= tr.mb_hi) return;
    const int64_t v0 = mbg * 16 + grp * 4;
    const int b = nb * 16 + l16;
    if (b >= p.B) return;
    const float a4[4] = {pend[nb][0], pend[nb][1], pend[nb][2], pend[nb][3]};
    if (EPI == EPI_STORE) {
      float* dst = p.logits + (int64_t)b * p.ldl + v0;
      if (v0 + 3 < p.V) {
        *(f32x4_t*)dst = pend[nb];
      } else {
        for (int i = 0; i < 4; ++i)
          if (v0 + i < p.V) dst[i] = a4[i];
      }
    } else if (EPI == EPI_TOPK) {
      topk_quad(p, (int)v0, a4, mask_bits4<MASKED>(p, mask_lds, mw_lo, p.vocab_offset + v0, b), tk[nb]);
    } else {
      const uint32_t bits = mask_bits4<MASKED>(p, mask_lds, mw_lo, p.vocab_offset + v0, b);
      f32x4_t g;
      if (NOISE_LDS)
        g = *(const f32x4_t*)(noise_lds + b * p.noise_pitch + (int)(v0 - tr.mb_lo * 16));
      else
        g = noise_quad(p, (int)(p.vocab_offset + v0), b);
      epilogue_quad<EPI>(p, (int)v0, a4, g, bits, bv[nb], bi[nb], lm[nb], ls[nb]);
    }
  };

  // NB <= 2: deferred (see above).  NB = 4: the block is finished at its end
  // (measured no slower, and it leaves the registers to the operand pipeline).
  constexpr bool kDefer = NB <= 2;
  // pblk: the wave's previous block (-1 if none); cblk: the block just completed
  auto body_b = [&](const u32x4_t (&cur)[8], const unsigned char* hbase, int sbc, int64_t pblk, int t) {
    compute(cur, hbase, sbc);
    if (kDefer && pblk >= 0 && t < NB) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (nb == t) finish_nb(pblk, nb);
    }
  };
  auto block_end = [&](int64_t cblk, int64_t pblk) {
    if (kDefer && pblk >= 0 && p.nsub < NB) {  // fewer sub-blocks per block than N-blocks
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (nb >= p.nsub) finish_nb(pblk, nb);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      pend[nb] = acc[nb];
      acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (!kDefer) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) finish_nb(cblk, nb);
    }
  };

  int64_t last_blk;
  // blocks on demand with H resident (the top-k merge rescores whole tiles, so
  // it does not need to know which wave took which block)
  if constexpr (RESIDENT && FAST) {
    __shared__ int next_blk;
    last_blk = stream_driver_dynamic<RING, LAYOUT>(p, tr, smem, &next_blk, body_b, block_end, pre);
  } else {
    // fixed rounds: wave w takes block mb_lo + 8r + w in round r
    auto blk_of = [&](int r) { return tr.mb_lo + (int64_t)r * kWaves + wave; };
    auto body = [&](const u32x4_t (&cur)[8], const unsigned char* hbase, int sbc, int r, int t) {
      body_b(cur, hbase, sbc, r > 0 ? blk_of(r - 1) : (int64_t)-1, t);
    };
    auto round_end = [&](int r) { block_end(blk_of(r), r > 0 ? blk_of(r - 1) : (int64_t)-1); };
    stream_driver<FAST, RESIDENT, RING, LAYOUT>(p, tr, smem, body, round_end, pre);
    last_blk = tr.rounds > 0 ? blk_of(tr.rounds - 1) : (int64_t)-1;
  }
  if (kDefer && last_blk >= 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) finish_nb(last_blk, nb);
  }
  if (EPI == EPI_STORE) return;
  if (EPI == EPI_TOPK) {
    finish_wave_topk<NB>(p, smem, tk);
    return;
  }
  finish_wave_tile<EPI, NB>(p, smem, bv, bi, lm, ls);
}


// ---------------------------------------------------------------------------
// Chunk-outer MFMA kernel, for H that does not fit in LDS (fast shapes: chunks
// of exactly kFastRingChunked 256-wide sub-blocks).  The round-major kernel
// restages every H chunk once per round; here each pass over the tile covers
// RM rounds and loops chunk-outer: for each chunk c, for each round r < RM,
// for each sub-block s of the chunk, W[block of round r][k range (c, s)] is
// streamed and accumulated into acc[r] (RM * NB accumulator sets stay in
// registers).  Each chunk is thereby staged once per pass instead of once per
// round.  Rounds past the wave's last block re-read that block (recently
// fetched, so an L2 hit) and their results are dropped.  With a sampling
// epilogue each round of a pass is finished (scale, mask, noise, argmax) right
// after its part of the last chunk, while the loads of the next round are in
// flight; stored logits are written at the end of the pass.
// ---------------------------------------------------------------------------
template <int NB, int EPI, bool MASKED, int RM>
__global__ void __launch_bounds__(kThreads) fmms_kouter_kernel(const StreamParams p) {
  constexpr int LAYOUT = EPI == EPI_TOPK ? kLayoutKouterTopk : kLayoutKouter;
  if constexpr (EPI == EPI_GROUP) {
    // the answer is the same in every lane; readfirstlane tells the compiler so
    if (p.ready && !__builtin_amdgcn_readfirstlane((int)group_published(p))) return;
  }
  static_assert(kFastRingChunked == 2, "two sub-blocks per chunk, two register buffers");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block indices and bases stay scalar
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range(p);
  const int rs = p.h_rowstride;
  const int bufbytes = p.h_rows * rs;
  uint32_t* mask_lds = (uint32_t*)(smem + p.mask_lds_off);
  const int64_t mw_lo = mask_w_lo(p, tr);
  if (MASKED) mask_stage(p, tr, mask_lds);  // made visible by the first barrier below
  int hoff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = nb * 16 + l16;
    hoff[nb] = lane_base<LAYOUT>(grp) + (row < p.B ? row : p.h_rows - 1) * rs;
  }
  float bv[NB], lm[NB], ls[NB];
  int32_t bi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = -INFINITY;
    bi[nb] = -1;
    lm[nb] = -INFINITY;
    ls[nb] = 0.0f;
  }
  f32x4_t acc[RM][NB];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  TopkList tk[NB];  // EPI_TOPK only
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) topk_init(tk[nb]);

  const int nchunk = p.nchunk;
  const int npass = (tr.rounds + RM - 1) / RM;
  // the wave's last block of the tile (the clamp target of empty rounds)
  const int64_t nown = tr.mb_hi - tr.mb_lo - wave > 0 ? (tr.mb_hi - tr.mb_lo - wave + kWaves - 1) / kWaves : 0;
  const int64_t last_blk = nown > 0 ? tr.mb_lo + (nown - 1) * kWaves + wave : tr.mb_hi - 1;
  auto blk = [&](int pass, int r) {
    const int64_t mb = tr.mb_lo + (int64_t)(pass * RM + r) * kWaves + wave;
    return mb < tr.mb_hi ? mb : last_blk;
  };
  const WLane wl = w_lane<LAYOUT>(p, tr, l16, grp);
  auto load = [&](u32x4_t (&buf)[8], int64_t mb, int sb) { w_load8<LAYOUT>(p, tr, wl, mb, sb, buf); };
  auto compute = [&](const u32x4_t (&cur)[8], const unsigned char* hb, f32x4_t (&a)[NB]) {
    u32x4_t h0[NB], h1[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) h0[nb] = *(const u32x4_t*)(hb + hoff[nb]);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) h1[nb] = *(const u32x4_t*)(hb + hoff[nb] + (j + 1) * lane_step<LAYOUT>());
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[j]),
                                                        __builtin_bit_cast(bf16x8_t, h0[nb]), a[nb], 0, 0, 0);
      if (j + 2 < 8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) h0[nb] = *(const u32x4_t*)(hb + hoff[nb] + (j + 2) * lane_step<LAYOUT>());
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[j + 1]),
                                                        __builtin_bit_cast(bf16x8_t, h1[nb]), a[nb], 0, 0, 0);
    }
  };
  auto finish = [&](int pass, int r, const f32x4_t (&a)[NB]) {
    const int64_t mbg = tr.mb_lo + (int64_t)(pass * RM + r) * kWaves + wave;
    if (mbg >= tr.mb_hi) return;
    const int v0 = (int)(mbg * 16) + grp * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + l16;
      if (b >= p.B) continue;
      if (EPI == EPI_STORE) {
        float* dst = p.logits + (int64_t)b * p.ldl + v0;
        if (v0 + 3 < p.V) {
          *(f32x4_t*)dst = a[nb];
        } else {
          for (int i = 0; i < 4; ++i)
            if (v0 + i < p.V) dst[i] = a[nb][i];
        }
      } else if (EPI == EPI_TOPK) {
        const float a4[4] = {a[nb][0], a[nb][1], a[nb][2], a[nb][3]};
        topk_quad(p, v0, a4, mask_bits4<MASKED>(p, mask_lds, mw_lo, p.vocab_offset + v0, b), tk[nb]);
      } else {
        const float a4[4] = {a[nb][0], a[nb][1], a[nb][2], a[nb][3]};
        const uint32_t bits = mask_bits4<MASKED>(p, mask_lds, mw_lo, p.vocab_offset + v0, b);
        const f32x4_t g = noise_quad(p, (int)(p.vocab_offset + v0), b);
        epilogue_quad<EPI>(p, (int)v0, a4, g, bits, bv[nb], bi[nb], lm[nb], ls[nb]);
      }
      __builtin_amdgcn_sched_barrier(0);  // one N-block's noise at a time (register pressure)
    }
  };

  if (tr.rounds > 0) {
    // zero rows (the padding lanes' row) of both buffers, then chunk 0
    for (int i = tid; i < (p.h_rows - p.B) * 64; i += kThreads) {
      const int row = p.B + i / 64, q = i % 64;
      *(u32x4_t*)(smem + row * rs + q * 16) = u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t*)(smem + bufbytes + row * rs + q * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
    // Each workgroup takes the chunks in a rotated order (from chunk blockIdx mod
    // nchunk), so that workgroups stream different k ranges of their W rows and
    // copy different H chunks at any one time.  In the same order for every
    // workgroup, small decode (d=2048) at B=64 took 140 us instead of 115 on
    // MI355X.  The masked kernels keep the plain order: the masked workload
    // (d=5120, B=32) was 1% slower rotated.
    const int rot = MASKED ? 0 : (int)(blockIdx.x % (unsigned)nchunk);
    h_chunk_dma<2 * NB>(p, rot, smem);
    int64_t rowp[RM];  // the wave's block in each round of the pass
#pragma unroll
    for (int r = 0; r < RM; ++r) rowp[r] = blk(0, r);
    u32x4_t buf[2][8];
    load(buf[0], rowp[0], rot * 2);
    // the first W item is in flight behind the chunk-0 copies: once at most its
    // 8 loads remain (vmcnt 8), this wave's copies have landed
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xF78);
    __syncthreads();
    int cc = 0;  // chunks consumed
    for (int pass = 0; pass < npass; ++pass) {
      // Waves own RM or RM - 1 blocks in a pass (tiles differ by at most one
      // block); a wave without a block in the pass's last round skips that
      // round instead of re-reading data: its round RM - 2 goes straight on to
      // the next chunk.  Both paths leave the same 8 loads in flight into the
      // same registers, so the wait counts agree where they join.
      const bool last_on = nown >= (int64_t)(pass + 1) * RM;
      for (int cpos = 0; cpos < nchunk; ++cpos) {
        const int c = cpos + rot < nchunk ? cpos + rot : cpos + rot - nchunk;  // this chunk
        const unsigned char* hb = smem + (cc & 1) * bufbytes;
        const int nc = c + 1 < nchunk ? c + 1 : 0;  // the chunk staged next
        const bool last_c = cpos + 1 == nchunk;     // the pass's k reduction completes here
        const int np = last_c && pass + 1 < npass ? pass + 1 : pass;
        const int64_t next_row = last_c ? blk(np, 0) : rowp[0];  // first item of the next chunk
        const int next_sb = last_c ? rot * 2 : nc * 2;
        // In the last chunk each round is finished right after its compute.  The
        // finish is long ALU work, so the second sub-block of the next round is
        // loaded into the buffer just freed before it: two items stay in flight
        // through the finish instead of one, and that round skips its own load.
        const bool early = EPI != EPI_STORE && last_c;
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          if (r == RM - 1 && RM > 1 && !last_on) break;
          // Waves w and w + 4 share a SIMD, and the older one wins its issue
          // arbitration: left alone, waves 0-3 finished each chunk ~8 us ahead
          // of waves 4-7 and then idled at the chunk barrier (mid decode B=64,
          // 23 us chunks).  The higher priority goes to the two in turn, round
          // by round, so that both keep pace.
          if (((r ^ (wave >> 2)) & 1) != 0)
            __builtin_amdgcn_s_setprio(1);
          else
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            // the W item after (r, sb): same round's next sub-block, the next
            // round's first one, or the first one of the next chunk / pass
            if (sb == 0) {
              if (!(early && r > 0)) load(buf[1], rowp[r], c * 2 + 1);
            } else if (r + 2 < RM || (r + 2 == RM && RM > 1)) {
              if (r + 2 == RM)  // the next round is the last one: it may be skipped
                load(buf[0], last_on ? rowp[r + 1] : next_row, last_on ? c * 2 : next_sb);
              else
                load(buf[0], rowp[r + 1], c * 2);
            } else {
              load(buf[0], next_row, next_sb);
            }
            if (r == 0 && sb == 0) h_chunk_dma<2 * NB>(p, nc, smem + ((cc + 1) & 1) * bufbytes);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf[sb], hb + sb * 512, acc[r]);
          }
          // after the pass's last chunk, round r is complete: finish it while
          // the next item's loads are in flight (sampling epilogues; storing
          // the logits is cheap and is left to the end of the pass, which
          // keeps more rounds within the register budget)
          if (EPI != EPI_STORE && last_c) {
            // round r + 1 runs in this chunk unless it is a skipped last round
            if (r + 1 < RM && (r + 2 < RM || last_on)) load(buf[1], rowp[r + 1], c * 2 + 1);
            __builtin_amdgcn_sched_barrier(0);
            finish(pass, r, acc[r]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the chunk's copies were issued before the last W item (8 loads), so
        // at most those 8 loads may still be outstanding: vmcnt(8)
        __builtin_amdgcn_s_waitcnt(0xF78);
        __syncthreads();
        ++cc;
      }
      if (EPI == EPI_STORE) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          finish(pass, r, acc[r]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (pass + 1 < npass) {
#pragma unroll
        for (int r = 0; r < RM; ++r) rowp[r] = blk(pass + 1, r);
      }
    }
  }
  if (EPI == EPI_STORE) return;
  if (EPI == EPI_TOPK) {
    finish_wave_topk<NB>(p, smem, tk);
    return;
  }
  finish_wave_tile<EPI, NB>(p, smem, bv, bi, lm, ls);
}

// ---------------------------------------------------------------------------
// Wide kernel: 65 .. 256 batch rows of the plain sampler in one pass over W.
// At these batch sizes each W byte carries 4 to 16 times the MFMA work of a
// decode step, and operand reuse in registers decides the speed: a wave keeps
// an 80 x 16 NB block of logits in accumulators (5 vocab blocks of 16 rows
// against NB batch blocks of 16 columns), so every W fragment feeds NB MFMAs
// and every H fragment read from LDS feeds five.  At 256 rows and the MFMA
// peak that is about 51 bytes per clock of LDS reads and 16 of W loads per CU.
// Four waves, one per SIMD (the accumulators take up to 320 registers: all
// 256 AGPRs and 64 VGPRs at 256 rows), run passes of up to 20 vocab blocks:
// the tile's blocks are split into as few near-equal passes as that allows
// (a tile of 37 blocks: two), each wave taking a quarter of a pass (block
// slots past a wave's count compute on repeated rows and are discarded).
// Every pass reads all of H again, so the passes per tile set the H traffic.
// H comes through LDS in k-chunks of 32 KSTEPS, three buffers, copied
// straight from global memory; W goes straight into registers, each chunk's
// item two chunks ahead of its MFMAs.  The chunk order is rotated per
// workgroup, as in the chunk-outer kernel.
// ---------------------------------------------------------------------------
template <int NB>
struct WideGeom {
  static constexpr int KSTEPS = wide_ksteps(NB);
  static constexpr int PIECES = wide_pieces(NB);  // 16-byte pieces per LDS row, the last one padding
  static constexpr int ROWBYTES = PIECES * 16;
  static constexpr int BUFBYTES = wide_bufbytes(NB);
  static constexpr int RUNS_W = (NB * 16 * PIECES / 64 + kWideWaves - 1) / kWideWaves;  // copies per wave
  static constexpr int MW = wide_mw(NB);                                                  // vocab block slots per wave
  static constexpr int NW = MW * KSTEPS;                                                  // W loads per item
  static_assert(NB * 16 * PIECES % 64 == 0, "a buffer is a whole number of 1 KB runs");
};

// H k-chunk c (k in [32 KSTEPS c, 32 KSTEPS (c + 1))) into buf, all 16 NB
// rows, as whole 1 KB runs of 16-byte pieces (an LDS-direct load writes 64
// consecutive pieces): piece j of the buffer is piece j mod PIECES of row
// j / PIECES, a row's last piece being padding (a copy of its first).  Rows
// past B repeat row B - 1, so that a lane's H offsets are affine in its batch
// block.  Every wave issues RUNS_W copies; runs past the last repeat it,
// writing the same bytes to the same place.
// This lane's source offset (bytes from chunk 0 of H) of its piece of each of
// its RUNS_W runs: the same for every chunk.
template <int NB>
__device__ __forceinline__ void h_wide_offsets(const StreamParams& p, uint32_t (&hsrc)[WideGeom<NB>::RUNS_W]) {
  using G = WideGeom<NB>;
  constexpr int nrun = NB * 16 * G::PIECES / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int k = 0; k < G::RUNS_W; ++k) {
    const int r0 = wave + k * kWideWaves;
    const int run = r0 < nrun ? r0 : nrun - 1;
    const int piece = run * 64 + lane;
    const int row = piece / G::PIECES, col = piece - row * G::PIECES;
    const int srow = row < p.B ? row : p.B - 1;
    const int scol = col < G::PIECES - 1 ? col : 0;
    hsrc[k] = (uint32_t)(srow * p.ldh + scol * 8) * 2u;
  }
}

// Run k of this wave's copies of H chunk c into buf.
template <int NB>
__device__ __forceinline__ void h_wide_run(const StreamParams& p, int c, unsigned char* buf,
                                           const uint32_t (&hsrc)[WideGeom<NB>::RUNS_W], int k) {
  using G = WideGeom<NB>;
  constexpr int nrun = NB * 16 * G::PIECES / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = wave + k * kWideWaves;
  const int run = r0 < nrun ? r0 : nrun - 1;
  lds_copy16_s((const char*)p.H + c * (64 * G::KSTEPS), hsrc[k], buf + run * 1024);
}

template <int NB>
__device__ __forceinline__ void h_wide_dma(const StreamParams& p, int c, unsigned char* buf,
                                           const uint32_t (&hsrc)[WideGeom<NB>::RUNS_W]) {
#pragma unroll
  for (int k = 0; k < WideGeom<NB>::RUNS_W; ++k) h_wide_run<NB>(p, c, buf, hsrc, k);
}

// The loads of one W item: per block slot, a scalar base (the block's rows
// at the chunk's k offset) and the lane's offset in it.
template <int MW>
struct WideItem {
  const char* base[MW];
  uint32_t off[MW];
};

// One 16x16x32 bf16 MFMA, acc += a * b, written in assembly with its
// accumulator in AGPRs (ag, a constant after unrolling) or VGPRs.  The wide kernel's 80 accumulator
// blocks at 256 rows need both register files; with the builtin, the compiler
// gives every MFMA of a function accumulators of one class and copied the
// rest across each chunk.  The compiler does not see these as MFMAs, so it
// inserts no wait states for them: each accumulator is touched once per
// chunk (dozens of MFMAs apart), and the kernel spaces the last MFMAs of a
// pass from any vector instruction that reads their results (s_nop).
__device__ __forceinline__ void mfma_bf16_asm(bool ag, f32x4_t& acc, const u32x4_t a, const u32x4_t b) {
  if (ag)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// The MFMAs of one k-chunk, group by group (a group: one 32-wide k-step
// against four batch blocks, for the wave's MW vocab block slots), with the
// vector-memory work of a later chunk spread over the groups: the copies of
// H chunk c3 into hbuf3, then the W item `it` into dst.  Issued in one burst,
// those loads held the wave up for as long as the CU's address unit took to
// accept them, with no MFMA in flight; spread out, each slice issues while
// the matrix core works through the previous group.  Each group's H fragments
// are read one group ahead.  Block slots past the wave's block count compute
// on repeated rows and are discarded: a run-time skip would split the
// accumulators' live ranges over two paths, which the register allocator
// answered with a copy of all of them per chunk.
template <int NB, int GI>
__device__ __forceinline__ void wide_groups(const u32x4_t (&w)[wide_mw(NB)][wide_ksteps(NB)], const unsigned char* hb,
                                            f32x4_t (&acc)[wide_mw(NB)][NB], u32x4_t (&h)[2][4], const StreamParams& p, int c3,
                                            unsigned char* hbuf3, const uint32_t (&hsrc)[WideGeom<NB>::RUNS_W],
                                            const WideItem<wide_mw(NB)>& it,
                                            u32x4_t (&dst)[wide_mw(NB)][wide_ksteps(NB)]) {
  constexpr int KS = wide_ksteps(NB), MW = wide_mw(NB), NG = NB / 4, NGRP = KS * NG;
  constexpr int BLK = 16 * WideGeom<NB>::ROWBYTES;  // LDS bytes between batch blocks
  constexpr int RUNS = WideGeom<NB>::RUNS_W, PIECES = RUNS + MW * KS;
  if constexpr (GI < NGRP) {
    constexpr int j0 = GI * PIECES / NGRP, j1 = (GI + 1) * PIECES / NGRP;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      if (j < RUNS) {
        h_wide_run<NB>(p, c3, hbuf3, hsrc, j);
      } else {
        const int m = (j - RUNS) / KS, e = (j - RUNS) % KS;
        dst[m][e] = *(const u32x4_t*)(it.base[m] + it.off[m] + e * 64);
      }
    }
    if constexpr (GI + 1 < NGRP) {
      constexpr int e1 = (GI + 1) / NG, ng1 = (GI + 1) % NG;
#pragma unroll
      for (int q = 0; q < 4; ++q) h[(GI + 1) & 1][q] = *(const u32x4_t*)(hb + (ng1 * 4 + q) * BLK + e1 * 64);
    }
    constexpr int e = GI / NG, ng = GI % NG;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) mfma_bf16_asm(m * NB < 64, acc[m][ng * 4 + q], w[m][e], h[GI & 1][q]);
    }
    __builtin_amdgcn_sched_barrier(0);
    wide_groups<NB, GI + 1>(w, hb, acc, h, p, c3, hbuf3, hsrc, it, dst);
  }
}

// Pass q of a tile: the tile's blocks split into npass near-equal passes of
// at most kWideWaves * MW blocks; wave w's first block and block count in it
// (the lower waves take one more where the pass does not divide by four; none
// past the last pass, where the tile's last block stands in for the loads).
__device__ __forceinline__ void wide_geom(int mb_lo, int mb_hi, int q, int npass, int wave, int& mb0, int& mw) {
  if (q >= npass) {
    mb0 = mb_hi - 1;
    mw = 0;
    return;
  }
  const int nblk = mb_hi - mb_lo;
  const int lo = mb_lo + q * nblk / npass;
  const int n = mb_lo + (q + 1) * nblk / npass - lo;
  const int base = n >> 2, extra = n & 3;
  mw = base + (wave < extra ? 1 : 0);
  mb0 = lo + wave * base + (wave < extra ? wave : extra);
}

// The W item of chunk c of pass q: for block slots m = 0 .. MW - 1, the lane's 16
// bytes of each of the chunk's k-steps (kouter layout: lane group g feeds k
// values 8 g .. 8 g + 7 of each 32-wide step).  Slots past the wave's block
// count repeat its last block (the tile's last with none), so that every item
// issues the same loads; rows of the tile's last block are clamped to its end
// (off_delta).
template <int NB>
__device__ __forceinline__ WideItem<wide_mw(NB)> wide_item(const StreamParams& p, int mb_lo, int mb_hi, int npass,
                                                           int wave, uint32_t off_full, uint32_t off_delta, int q,
                                                           int c) {
  int mb0, mw;
  wide_geom(mb_lo, mb_hi, q, npass, wave, mb0, mw);
  WideItem<wide_mw(NB)> it;
#pragma unroll
  for (int m = 0; m < wide_mw(NB); ++m) {
    const int mb = mw == 0 ? mb_hi - 1 : mb0 + (m < mw ? m : mw - 1);
    it.base[m] = (const char*)p.W + (int64_t)mb * 16 * p.ldw * 2 + c * (wide_ksteps(NB) * 64);
    it.off[m] = off_full + (mb == mb_hi - 1 ? off_delta : 0u);
  }
  return it;
}

template <int NB>
__device__ __forceinline__ void wide_wload(const WideItem<wide_mw(NB)>& it,
                                           u32x4_t (&dst)[wide_mw(NB)][wide_ksteps(NB)]) {
#pragma unroll
  for (int m = 0; m < wide_mw(NB); ++m)
#pragma unroll
    for (int e = 0; e < wide_ksteps(NB); ++e) dst[m][e] = *(const u32x4_t*)(it.base[m] + it.off[m] + e * 64);
}

template <int NB>
__global__ void __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
fmms_wide_kernel(const StreamParams p) {
  using G = WideGeom<NB>;
  constexpr int KS = G::KSTEPS, MW = G::MW;
  constexpr int RING = wide_ring(NB), LEAD = wide_lead(NB);
  static_assert(LEAD >= 2 && LEAD < RING, "an item's slot is free once its chunk's MFMAs ran");
  // The wait at the start of item t leaves at most WAIT loads and copies in
  // flight.  The copies of chunk t + 1 went out in item t - 1, before the W
  // items of chunks t + LEAD - 1 and, from item t - 1 on, t + LEAD ... what
  // chunk t needs is everything up to them.  The compiler counts only the W
  // loads (not the copies), and unless the wait also leaves at most the W
  // items after chunk t's in flight by its count, it adds a wait of its own
  // before the MFMAs that drains more; so the wait is the smaller of the two.
  constexpr int NEED = LEAD == 2 ? G::NW + G::RUNS_W : 2 * G::NW + G::RUNS_W;
  constexpr int WAIT = NEED < (LEAD - 1) * G::NW ? NEED : (LEAD - 1) * G::NW;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range(p);
  // the tile's blocks as wave-uniform 32-bit values (block counts are far below
  // 2^31), so that the W addressing runs on the scalar unit
  const int mb_lo = __builtin_amdgcn_readfirstlane((int)tr.mb_lo);
  const int mb_hi = __builtin_amdgcn_readfirstlane((int)tr.mb_hi);
  const int nchunk = p.d / (32 * KS);
  const int npass = (mb_hi - mb_lo + kWideWaves * MW - 1) / (kWideWaves * MW);
  const int rot = (int)(blockIdx.x % (unsigned)nchunk);
  // this lane's H fragment in batch block 0 (the others follow at fixed
  // offsets: rows past B hold copies of row B - 1)
  const int hoff = (l16 < p.B ? l16 : p.B - 1) * G::ROWBYTES + grp * 16;
  const WLane wl = w_lane<kLayoutKouter>(p, tr, l16, grp);
  const uint32_t off_full = wl.full, off_delta = wl.last - wl.full;  // rows of the tile's last block are clamped
  float bv[NB], lm[NB], ls[NB];  // lm, ls: unused by the plain sampler
  int32_t bi[NB];
  f32x4_t acc[MW][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = -INFINITY;
    bi[nb] = -1;
    lm[nb] = -INFINITY;
    ls[nb] = 0.0f;
#pragma unroll
    for (int m = 0; m < MW; ++m) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  u32x4_t wb[RING][MW][KS];

  // chunks 0 and 1's H, then the W items of chunks 0 .. LEAD-1 (all of pass 0:
  // nchunk is a multiple of RING)
  uint32_t hsrc[G::RUNS_W];
  h_wide_offsets<NB>(p, hsrc);
  h_wide_dma<NB>(p, rot, smem, hsrc);
  h_wide_dma<NB>(p, rot + 1 < nchunk ? rot + 1 : 0, smem + G::BUFBYTES, hsrc);
  // (in chunk order: the compiler's wait for an item's registers counts the
  // loads issued after it)
#pragma unroll
  for (int j = 0; j < LEAD; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    wide_wload<NB>(wide_item<NB>(p, mb_lo, mb_hi, npass, wave, off_full, off_delta, 0,
                                 rot + j < nchunk ? rot + j : rot + j - nchunk),
                   wb[j]);
  }
  __builtin_amdgcn_sched_barrier(0);
  int hcur = 0;  // LDS buffer of the current chunk (chunk t uses buffer t mod 3)
  for (int q = 0; q < npass; ++q) {
    int mb0, mw;
    wide_geom(mb_lo, mb_hi, q, npass, wave, mb0, mw);
    for (int cpos = 0; cpos < nchunk; cpos += RING) {
      // the RING items of the register ring, written out so that every index
      // into the ring and the accumulators is a constant from the start
#define FS_WIDE_ITEM(r)                                                                    \
  if constexpr ((r) < RING) {                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(WAIT));                                          \
    __syncthreads();                                                                       \
    const int n2 = cpos + (r) + LEAD;                                                      \
    const int q2 = n2 >= nchunk ? q + 1 : q;                                               \
    const int cp2 = n2 >= nchunk ? n2 - nchunk : n2;                                       \
    const int c2 = cp2 + rot < nchunk ? cp2 + rot : cp2 + rot - nchunk;                    \
    const int n3 = cpos + (r) + 2;                                                         \
    const int cp3 = n3 >= nchunk ? n3 - nchunk : n3;                                       \
    const int c3 = cp3 + rot < nchunk ? cp3 + rot : cp3 + rot - nchunk;                    \
    const WideItem<MW> it = wide_item<NB>(p, mb_lo, mb_hi, npass, wave, off_full, off_delta, q2, c2); \
    const unsigned char* hb = smem + hcur * G::BUFBYTES + hoff;                            \
    u32x4_t h[2][4];                                                                       \
    _Pragma("unroll") for (int qq = 0; qq < 4; ++qq) h[0][qq] =                             \
        *(const u32x4_t*)(hb + qq * 16 * G::ROWBYTES);                                     \
    wide_groups<NB, 0>(wb[(r) % RING], hb, acc, h, p, c3,                                  \
                       smem + (hcur == 0 ? 2 : hcur - 1) * G::BUFBYTES, hsrc, it,          \
                       wb[((r) + LEAD) % RING]);                                           \
    hcur = hcur == 2 ? 0 : hcur + 1;                                                       \
    if constexpr ((r) == RING - 1) { /* results read by vector code after the loop */     \
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");                          \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
  }
      // Each item t: everything but the last three batches issued (chunk
      // t + LEAD - 1's W item, chunk t + 2's copies, chunk t + LEAD's W item)
      // has landed, which covers this wave's copies of chunk t + 1 and its W
      // item of chunk t + 1 (the W loads are visible to the compiler, the
      // copies are not, so its own waits only ever cover more); the barrier
      // makes every wave's copies of chunk t visible and frees buffer
      // (t + 2) mod 3; chunk t + 2's copies and chunk t + LEAD's W item go out;
      // chunk t's MFMAs run.
      static_assert(RING <= 8, "items written out below");
      FS_WIDE_ITEM(0)
      FS_WIDE_ITEM(1)
      FS_WIDE_ITEM(2)
      FS_WIDE_ITEM(3)
      FS_WIDE_ITEM(4)
      FS_WIDE_ITEM(5)
      FS_WIDE_ITEM(6)
      FS_WIDE_ITEM(7)
#undef FS_WIDE_ITEM
    }
    // the pass's epilogue, one vocab block slot at a time (written out: see
    // the items above); the next two chunks' copies and W loads are in flight
#define FS_WIDE_EPI(m)                                                                            \
  if constexpr ((m) < MW) {                                                                       \
    if ((m) < mw) {                                                                               \
      const int v0 = (int)((mb0 + (m)) * 16) + grp * 4;                                           \
      int lb = l16; /* opaque here, so that no row's noise terms are kept across the pass */      \
      asm volatile("" : "+v"(lb));                                                                \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                         \
        const int b = nb * 16 + lb;                                                               \
        if (b < p.B) {                                                                            \
          const float a4[4] = {acc[m][nb][0], acc[m][nb][1], acc[m][nb][2], acc[m][nb][3]};       \
          const f32x4_t g = noise_quad<false>(p, (int)(p.vocab_offset + v0), b);                  \
          epilogue_quad<EPI_FLAT>(p, v0, a4, g, 0xFu, bv[nb], bi[nb], lm[nb], ls[nb]);            \
        }                                                                                         \
        __builtin_amdgcn_sched_barrier(0); /* one quad's noise at a time (registers) */          \
      }                                                                                           \
    }                                                                                             \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};   \
  }
    FS_WIDE_EPI(0)
    FS_WIDE_EPI(1)
    FS_WIDE_EPI(2)
    FS_WIDE_EPI(3)
    FS_WIDE_EPI(4)
    FS_WIDE_EPI(5)
    FS_WIDE_EPI(6)
    FS_WIDE_EPI(7)
    static_assert(MW <= 8, "block slots written out above");
#undef FS_WIDE_EPI
  }
  // the copies past the last chunk write LDS: all of them land before it is reused
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  finish_wave_tile<EPI_FLAT, NB, kWideWaves>(p, smem, bv, bi, lm, ls);
}

// ---------------------------------------------------------------------------
// Dot-product streaming kernel for small batches (B <= BD <= 2): the same W
// stream, with bf16 pair dot products on the vector ALU against H rows read
// from LDS (one address per 16-lane group, i.e. broadcast reads).  The four
// lane groups are summed (two cross-lane steps) in the deferred epilogue;
// lane (r, g) then handles row r for batch row g.
// ---------------------------------------------------------------------------
// The bf16 pairs are taken with shufflevector from the 8-wide bf16 view: a
// bit_cast of each 32-bit vector element to bf16x2 is miscompiled by this
// toolchain (every call then reads element 0).
__device__ __forceinline__ float dot8(const u32x4_t w, const u32x4_t h, float c) {
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, h);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), c, false);
  return c;
}

template <int BD, int EPI, bool RESIDENT, bool FAST, bool MASKED,
          int RING = (RESIDENT ? kFastRingResident : kFastRingChunked)>
__global__ void __launch_bounds__(kThreads) fmms_dot_kernel(const StreamParams p) {
  static_assert(BD <= 2, "dot kernel handles at most 2 batch rows");
  if constexpr (EPI == EPI_GROUP) {
    // the answer is the same in every lane; readfirstlane tells the compiler so
    if (p.ready && !__builtin_amdgcn_readfirstlane((int)group_published(p))) return;
  }
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range(p);
  const int rs = p.h_rowstride;
  uint32_t* mask_lds = (uint32_t*)(smem + p.mask_lds_off);
  const int64_t mw_lo = mask_w_lo(p, tr);
  auto pre = [&]() {
    if (MASKED) mask_stage(p, tr, mask_lds);
  };

  float bv = -INFINITY, lm = -INFINITY, ls = 0.0f;
  int32_t bi = -1;
  float acc[BD], pend[BD];
#pragma unroll
  for (int b = 0; b < BD; ++b) {
    acc[b] = 0.0f;
    pend[b] = 0.0f;
  }

  auto compute = [&](const u32x4_t (&cur)[8], const unsigned char* hbase, int sbc) {
    const unsigned char* hb = hbase + sbc * 512 + lane_base<kLayoutDot>(grp);
    u32x4_t h0[BD], h1[BD];
#pragma unroll
    for (int b = 0; b < BD; ++b) h0[b] = *(const u32x4_t*)(hb + b * rs);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
#pragma unroll
      for (int b = 0; b < BD; ++b) h1[b] = *(const u32x4_t*)(hb + b * rs + (j + 1) * lane_step<kLayoutDot>());
      __builtin_amdgcn_sched_barrier(0);  // reads of step j + 1 stay ahead of the products of step j
#pragma unroll
      for (int b = 0; b < BD; ++b) acc[b] = dot8(cur[j], h0[b], acc[b]);
      if (j + 2 < 8) {
#pragma unroll
        for (int b = 0; b < BD; ++b) h0[b] = *(const u32x4_t*)(hb + b * rs + (j + 2) * lane_step<kLayoutDot>());
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < BD; ++b) acc[b] = dot8(cur[j + 1], h1[b], acc[b]);
    }
  };

  auto finish_round = [&](int rnd) {
    float x[BD];
#pragma unroll
    for (int b = 0; b < BD; ++b) {
      x[b] = pend[b] + __shfl_xor(pend[b], 16);
      x[b] += __shfl_xor(x[b], 32);
    }
    const int64_t mbg = tr.mb_lo + (int64_t)rnd * kWaves + wave;
    const int b = grp;
    if (mbg >= tr.mb_hi || b >= p.B || b >= BD) return;
    const int64_t v = mbg * 16 + l16;
    const int64_t gv = p.vocab_offset + v;
    const float xv = (BD == 1 || b == 0) ? x[0] : x[BD - 1];
    if (EPI == EPI_STORE) {
      if (v < p.V) p.logits[(int64_t)b * p.ldl + v] = xv;
      return;
    }
    const VRow vr = vrow_of(p, b);
    const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)(gv >> 2), vr.row, vr.step_lo, vr.step_hi);
    const uint32_t q = (uint32_t)(gv & 3);
    const uint32_t word = q == 0 ? r.w[0] : q == 1 ? r.w[1] : q == 2 ? r.w[2] : r.w[3];
    const bool ok = v < p.V && ((mask_bits4<MASKED>(p, mask_lds, mw_lo, gv & ~(int64_t)3, b) >> q) & 1u);
    const float sc = xv * p.inv_t;
    const float pv = ok ? sc + gumbel_from_bits(word) : -INFINITY;
    if (pv > bv) {
      bv = pv;
      bi = (int32_t)gv;
    }
    if (EPI == EPI_GROUP && ok) lse_push(lm, ls, sc);
  };

  auto body = [&](const u32x4_t (&cur)[8], const unsigned char* hbase, int sbc, int r, int t) {
    compute(cur, hbase, sbc);
    if (r > 0 && t == 0) finish_round(r - 1);
  };
  auto round_end = [&](int) {
#pragma unroll
    for (int b = 0; b < BD; ++b) {
      pend[b] = acc[b];
      acc[b] = 0.0f;
    }
  };

  stream_driver<FAST, RESIDENT, RING, kLayoutDot>(p, tr, smem, body, round_end, pre);
  if (tr.rounds > 0) finish_round(tr.rounds - 1);
  if (EPI == EPI_STORE) return;

  // Reduce over the 16 rows of each lane group.
#pragma unroll
  for (int off = 1; off <= 8; off <<= 1) {
    const float ov = __shfl_xor(bv, off);
    const int32_t oi = __shfl_xor(bi, off);
    merge_best(bv, bi, ov, oi);
    if (EPI == EPI_GROUP) {
      const float om = __shfl_xor(lm, off);
      const float os = __shfl_xor(ls, off);
      lse_merge(lm, ls, om, os);
    }
  }
  __syncthreads();
  float* sv = (float*)smem;
  int32_t* si = (int32_t*)(sv + kWaves * BD);
  float* sm = (float*)(si + kWaves * BD);
  float* ss = sm + kWaves * BD;
  if (l16 == 0 && grp < BD) {
    sv[wave * BD + grp] = bv;
    si[wave * BD + grp] = bi;
    sm[wave * BD + grp] = lm;
    ss[wave * BD + grp] = ls;
  }
  __syncthreads();
  publish_tile<EPI>(p, BD, sv, si, sm, ss);
}

// ---------------------------------------------------------------------------
// Launch of one streaming configuration (instantiated once per epilogue, each
// in its own translation unit).
// ---------------------------------------------------------------------------
// The dynamic-LDS limit of each kernel is raised to the full budget once per
// device (the attribute call is far slower than a launch).
template <typename K>
static hipError_t launch_with_lds(K kernel, int grid, int lds, hipStream_t stream, const StreamParams& p,
                                  int threads = kThreads) {
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, stream, p);
  return hipGetLastError();
}

template <int EPI, bool RES, bool FAST, bool MK, bool NZ>
static hipError_t launch_variant(const StreamParams& p, const StreamConfig& c, hipStream_t s) {
  const int g = p.n_tiles, L = c.lds_bytes;
  if (c.dot) {
    if constexpr (EPI == EPI_TOPK) return hipErrorInvalidValue;  // the top-k epilogue is MFMA-only
    switch (c.bd) {
      case 1: return launch_with_lds(fmms_dot_kernel<1, EPI, RES, FAST, MK>, g, L, s, p);
      case 2: return launch_with_lds(fmms_dot_kernel<2, EPI, RES, FAST, MK>, g, L, s, p);
      default: return hipErrorInvalidValue;
    }
  }
  switch (c.nb) {
    case 1: return launch_with_lds(fmms_mfma_kernel<1, EPI, RES, FAST, MK, NZ>, g, L, s, p);
    case 2: return launch_with_lds(fmms_mfma_kernel<2, EPI, RES, FAST, MK, NZ>, g, L, s, p);
    case 4: return launch_with_lds(fmms_mfma_kernel<4, EPI, RES, FAST, MK, NZ>, g, L, s, p);
    default: return hipErrorInvalidValue;
  }
}

template <int EPI, bool MK, int NB>
static hipError_t launch_kouter(const StreamParams& p, const StreamConfig& c, hipStream_t s) {
  const int g = p.n_tiles, L = c.lds_bytes;
  constexpr int cap = kouter_max_rounds(EPI, NB, MK);
  switch (c.rm) {
    case 1: return launch_with_lds(fmms_kouter_kernel<NB, EPI, MK, 1>, g, L, s, p);
    case 2: return launch_with_lds(fmms_kouter_kernel<NB, EPI, MK, 2>, g, L, s, p);
    case 3:
      if constexpr (cap >= 3) return launch_with_lds(fmms_kouter_kernel<NB, EPI, MK, 3>, g, L, s, p);
      break;
    case 4:
      if constexpr (cap >= 4) return launch_with_lds(fmms_kouter_kernel<NB, EPI, MK, 4>, g, L, s, p);
      break;
    case 5:
      if constexpr (cap >= 5) return launch_with_lds(fmms_kouter_kernel<NB, EPI, MK, 5>, g, L, s, p);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

// The noise table is planned only for the fast driver and the sampling epilogues.
template <int EPI, bool MK>
static hipError_t launch_masking(const StreamParams& p, const StreamConfig& c, hipStream_t s) {
  const bool res = p.nchunk == 1;
  if (c.nb > 4) {  // the wide kernel
    if constexpr (!MK && EPI == EPI_FLAT) {
      if (c.nb == 8) return launch_with_lds(fmms_wide_kernel<8>, p.n_tiles, c.lds_bytes, s, p, kWideWaves * 64);
      if (c.nb == 16) return launch_with_lds(fmms_wide_kernel<16>, p.n_tiles, c.lds_bytes, s, p, kWideWaves * 64);
    }
    return hipErrorInvalidValue;
  }
  constexpr bool kNoiseEpi = EPI == EPI_FLAT || EPI == EPI_GROUP;  // epilogues that may read a noise table
  if (c.rm > 0 && !c.dot) {
    switch (c.nb) {
      case 1: return launch_kouter<EPI, MK, 1>(p, c, s);
      case 2: return launch_kouter<EPI, MK, 2>(p, c, s);
      case 4: return launch_kouter<EPI, MK, 4>(p, c, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (c.fast) {
    if (kNoiseEpi && p.noise_pitch > 0 && !c.dot)
      return res ? launch_variant<EPI, true, true, MK, kNoiseEpi>(p, c, s)
                 : launch_variant<EPI, false, true, MK, kNoiseEpi>(p, c, s);
    return res ? launch_variant<EPI, true, true, MK, false>(p, c, s) : launch_variant<EPI, false, true, MK, false>(p, c, s);
  }
  return res ? launch_variant<EPI, true, false, MK, false>(p, c, s) : launch_variant<EPI, false, false, MK, false>(p, c, s);
}

// The stored-logits epilogue never reads the mask.
template <int EPI>
hipError_t launch_stream_epi(const StreamParams& p, const StreamConfig& c, hipStream_t s) {
  if (EPI != EPI_STORE && p.mask) return launch_masking<EPI, EPI != EPI_STORE>(p, c, s);
  return launch_masking<EPI, false>(p, c, s);
}

}  // namespace fsk
