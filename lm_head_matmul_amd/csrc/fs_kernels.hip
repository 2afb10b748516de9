// fs_kernels.hip -- FlashSampling kernels for MI355X (gfx950 / CDNA4).
//
// Fused LM-head matmul + sample (FMMS): logits are computed tile by tile on
// chip, Gumbel noise is added, each vocabulary tile keeps one (value, index)
// maximizer per row, and a small reduction over tiles yields the sample; the
// [B, V] logits never reach HBM.  Exact because argmax decomposes over a
// partition of the vocabulary.  [FlashSampling, arXiv 2603.15854, abstract;
// readus.org FlashSampling summary, section on the two-stage FMMS kernel]
//
// Layout on the device (one persistent workgroup of 8 waves per vocab tile):
//  * A tile is a contiguous, balanced range of 16-row vocab blocks.  Each round
//    a wave owns MB blocks (16 * MB rows) and streams their rows of W straight
//    from HBM into VGPRs in the MFMA operand layout: lane (r, g) = (lane % 16,
//    lane / 16) reads 128 contiguous bytes of row r per 256-wide k sub-block,
//    as eight 16-byte loads (k chunks 8g .. 8g + 7).  Eight MFMA k-steps then
//    consume chunk 8g + j from lane group g at step j; the same k permutation
//    is used for H, so each MFMA still sums over 32 matching k values.
//  * H (the small operand) sits in LDS: the whole [B, d] when it fits,
//    otherwise k-chunks double-buffered across the round, prefetched into
//    registers one chunk ahead.  Rows are padded by 16 bytes so the B-operand
//    reads of 16 lanes land in distinct banks.
//  * Epilogue per round, on the accumulators: scale by 1/T, mask, Philox4x32-10
//    noise (one call covers the four consecutive vocab ids a lane holds), argmax
//    update.  Per tile, the winners go to a [B, n_tiles] workspace; the last
//    workgroup to finish (device-scope ticket) reduces over tiles.
#include "fs_device.h"
#include "fs_kernels.h"

namespace fsk {

// ---------------------------------------------------------------------------
// Cross-tile reduction by the last workgroup to finish.
// ---------------------------------------------------------------------------
template <int EPI>
__device__ void finish_tiles(const int B, const int n_tiles, const float* __restrict__ ws_val,
                             const int32_t* __restrict__ ws_idx, const float* __restrict__ ws_m,
                             const float* __restrict__ ws_s, unsigned int* ticket, int32_t* out_idx,
                             GroupSummary* out_sum) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(n_tiles - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int b = wave; b < B; b += kWaves) {
    float v = -INFINITY, m = -INFINITY, s = 0.0f;
    int32_t i = -1;
    for (int t = lane; t < n_tiles; t += 64) {
      const int64_t o = (int64_t)b * n_tiles + t;
      merge_best(v, i, ws_val[o], ws_idx[o]);
      if (EPI == EPI_GROUP) lse_merge(m, s, ws_m[o], ws_s[o]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off);
      const int32_t oi = __shfl_xor(i, off);
      merge_best(v, i, ov, oi);
      if (EPI == EPI_GROUP) {
        const float om = __shfl_xor(m, off);
        const float os = __shfl_xor(s, off);
        lse_merge(m, s, om, os);
      }
    }
    if (lane == 0) {
      if (EPI == EPI_GROUP) {
        GroupSummary g;
        g.lse = (m == -INFINITY) ? -INFINITY : m + logf(s);
        g.pmax = v;
        g.arg = i;
        out_sum[b] = g;
      } else {
        out_idx[b] = i;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-wave results (already reduced inside the wave) sit in LDS scratch as
// [kWaves][Bp] (val, idx, m, s); reduce over waves and publish the tile's entry.
template <int EPI>
__device__ void publish_tile(const StreamParams& p, const int Bp, const float* sv, const int32_t* si, const float* sm,
                             const float* ss) {
  const int tile = blockIdx.x;
  for (int b = threadIdx.x; b < p.B; b += kThreads) {
    float v = -INFINITY, m = -INFINITY, s = 0.0f;
    int32_t i = -1;
    for (int w = 0; w < kWaves; ++w) {
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

template <int MB>
__device__ __forceinline__ TileRange tile_range(const StreamParams& p) {
  TileRange t;
  t.mb_lo = (int64_t)blockIdx.x * p.n_mblocks / p.n_tiles;
  t.mb_hi = (int64_t)(blockIdx.x + 1) * p.n_mblocks / p.n_tiles;
  constexpr int RB = kWaves * MB;
  t.rounds = (int)((t.mb_hi - t.mb_lo + RB - 1) / RB);
  return t;
}

// Loads one 256-wide k sub-block of the wave's MB vocab blocks in MFMA operand
// layout: lane (r, g) gets W[row r][sb*256 + 64 g .. + 64] as 8 x 16 bytes.
template <int MB>
__device__ __forceinline__ void load_w(u32x4_t (&wr)[MB][8], const StreamParams& p, const TileRange& tr, int wave,
                                       int l16, int grp, int it) {
  const int rnd = it / p.nsub;
  const int sb = it - rnd * p.nsub;
  const int kb = sb * 256 + grp * 64;
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int64_t mb = tr.mb_lo + (int64_t)rnd * (kWaves * MB) + wave * MB + j;
    if (mb < tr.mb_hi) {
      int64_t row = mb * 16 + l16;
      row = row < p.V ? row : p.V - 1;
      const u32x4_t* src = (const u32x4_t*)(p.W + row * p.ldw + kb);
      if (kb + 64 <= p.d) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wr[j][e] = src[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wr[j][e] = (kb + e * 8 < p.d) ? src[e] : u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wr[j][e] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// H chunk `cidx` (k in [cidx*cs*256, ...)) as 16-byte pieces: piece P = n * (cs*32) + q.
__device__ __forceinline__ u32x4_t h_piece(const StreamParams& p, int Bp, int cidx, int P) {
  const int per_row = p.cs * 32;
  const int n = P / per_row;
  const int q = P - n * per_row;
  const int k = cidx * p.cs * 256 + q * 8;
  if (n < p.B && k < p.d) return *(const u32x4_t*)(p.H + (int64_t)n * p.ldh + k);
  (void)Bp;
  return u32x4_t{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void h_store(const StreamParams& p, unsigned char* buf, int P, u32x4_t v) {
  const int per_row = p.cs * 32;
  const int n = P / per_row;
  const int q = P - n * per_row;
  *(u32x4_t*)(buf + n * p.h_rowstride + q * 16) = v;
}

// Stages the whole chunk (all pieces) directly.
__device__ void h_stage_all(const StreamParams& p, int Bp, int cidx, unsigned char* buf) {
  const int np = Bp * p.cs * 32;
  for (int P = threadIdx.x; P < np; P += kThreads) h_store(p, buf, P, h_piece(p, Bp, cidx, P));
}

__device__ __forceinline__ void h_prefetch(u32x4_t (&hs)[kMaxStagePieces], const StreamParams& p, int Bp, int cidx) {
  const int np = Bp * p.cs * 32;
#pragma unroll
  for (int i = 0; i < kMaxStagePieces; ++i) {
    const int P = threadIdx.x + i * kThreads;
    if (P < np) hs[i] = h_piece(p, Bp, cidx, P);
  }
}

__device__ __forceinline__ void h_commit(const u32x4_t (&hs)[kMaxStagePieces], const StreamParams& p, int Bp,
                                         unsigned char* buf) {
  const int np = Bp * p.cs * 32;
#pragma unroll
  for (int i = 0; i < kMaxStagePieces; ++i) {
    const int P = threadIdx.x + i * kThreads;
    if (P < np) h_store(p, buf, P, hs[i]);
  }
}

// Perturbed scores of the four consecutive vocab ids v0 .. v0+3 (local ids,
// v0 % 4 == 0) of row b, given their raw logits; updates the running maximizer
// (and the log-sum-exp state in grouped mode).  The scan order of a lane is
// increasing in v, so a strict comparison keeps the lowest id on ties.
template <int EPI>
__device__ __forceinline__ void epilogue_quad(const StreamParams& p, int64_t v0, int b, const float (&acc)[4],
                                              float& bv, int32_t& bi, float& lm, float& ls) {
  const int64_t gv0 = p.vocab_offset + v0;
  const int64_t grow = (int64_t)p.row_offset + b;
  const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)(gv0 >> 2), (uint32_t)grow, p.step_lo, p.step_hi);
  uint32_t bits = 0xFu;
  if (p.mask) bits = (p.mask[grow * p.ldm + (gv0 >> 5)] >> (uint32_t)(gv0 & 31)) & 0xFu;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = (v0 + i < p.V) && ((bits >> i) & 1u);
    const float s = acc[i] * p.inv_t;
    const float pv = ok ? s + gumbel_from_bits(r.w[i]) : -INFINITY;
    if (pv > bv) {
      bv = pv;
      bi = (int32_t)(gv0 + i);
    }
    if (EPI == EPI_GROUP && ok) lse_push(lm, ls, s);
  }
}

// ---------------------------------------------------------------------------
// MFMA streaming kernel (batch padded to 16 * NB columns).
// ---------------------------------------------------------------------------
template <int NB, int MB, int EPI>
__global__ void __launch_bounds__(kThreads) fmms_mfma_kernel(const StreamParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int Bp = NB * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range<MB>(p);
  const int nsub = p.nsub, cs = p.cs, nchunk = p.nchunk;
  const int total = tr.rounds * nsub;
  const int bufbytes = Bp * p.h_rowstride;

  float bv[NB], lm[NB], ls[NB];
  int32_t bi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = -INFINITY;
    bi[nb] = -1;
    lm[nb] = -INFINITY;
    ls[nb] = 0.0f;
  }
  f32x4_t acc[MB][NB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t hs[kMaxStagePieces];
  u32x4_t wa[MB][8], wb[MB][8];
  int cc = 0;  // chunks completed so far (selects the LDS buffer)

  auto compute = [&](const u32x4_t (&cur)[MB][8], const unsigned char* hbase, int sbc) {
    const unsigned char* hb = hbase + sbc * 512 + grp * 128 + l16 * p.h_rowstride;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4_t hv = *(const u32x4_t*)(hb + nb * 16 * p.h_rowstride + j * 16);
#pragma unroll
        for (int m = 0; m < MB; ++m)
          acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[m][j]),
                                                              __builtin_bit_cast(bf16x8_t, hv), acc[m][nb], 0, 0, 0);
      }
    }
  };

  auto epilogue = [&](int rnd) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t mbg = tr.mb_lo + (int64_t)rnd * (kWaves * MB) + wave * MB + m;
      if (mbg < tr.mb_hi) {
        const int64_t v0 = mbg * 16 + grp * 4;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int b = nb * 16 + l16;
          if (b < p.B) {
            const float a4[4] = {acc[m][nb][0], acc[m][nb][1], acc[m][nb][2], acc[m][nb][3]};
            if (EPI == EPI_STORE) {
              float* dst = p.logits + (int64_t)b * p.ldl + v0;
              if (v0 + 3 < p.V) {
                *(f32x4_t*)dst = acc[m][nb];
              } else {
                for (int i = 0; i < 4; ++i)
                  if (v0 + i < p.V) dst[i] = a4[i];
              }
            } else {
              epilogue_quad<EPI>(p, v0, b, a4, bv[nb], bi[nb], lm[nb], ls[nb]);
            }
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  auto step = [&](int it, const u32x4_t (&cur)[MB][8], u32x4_t (&nxt)[MB][8]) {
    const int rnd = it / nsub;
    const int sb = it - rnd * nsub;
    const int cidx = sb / cs;
    const int sbc = sb - cidx * cs;
    if (it + 1 < total) load_w<MB>(nxt, p, tr, wave, l16, grp, it + 1);
    const bool chunked = nchunk > 1;
    const bool last_chunk_overall = (rnd == tr.rounds - 1) && (cidx == nchunk - 1);
    if (chunked && sbc == 0 && !last_chunk_overall)
      h_prefetch(hs, p, Bp, cidx + 1 < nchunk ? cidx + 1 : 0);
    const int buf = (p.nbuf == 2) ? (cc & 1) : 0;
    compute(cur, smem + buf * bufbytes, sbc);
    if (chunked && (sbc == cs - 1 || sb == nsub - 1)) {
      if (!last_chunk_overall) {
        if (p.nbuf == 2) {
          h_commit(hs, p, Bp, smem + ((cc + 1) & 1) * bufbytes);
          __syncthreads();
        } else {
          __syncthreads();
          h_commit(hs, p, Bp, smem);
          __syncthreads();
        }
      }
      ++cc;
    }
    if (sb == nsub - 1) epilogue(rnd);
  };

  if (total > 0) {
    if (nchunk == 1) {
      h_stage_all(p, Bp, 0, smem);
    } else {
      h_prefetch(hs, p, Bp, 0);
      h_commit(hs, p, Bp, smem);
    }
    __syncthreads();
    load_w<MB>(wa, p, tr, wave, l16, grp, 0);
    for (int it = 0; it < total; it += 2) {
      step(it, wa, wb);
      if (it + 1 < total) step(it + 1, wb, wa);
    }
  }
  if (EPI == EPI_STORE) return;

  // Reduce inside the wave: lanes l16, l16 + 16, l16 + 32, l16 + 48 share a column.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ov = __shfl_xor(bv[nb], off);
      const int32_t oi = __shfl_xor(bi[nb], off);
      merge_best(bv[nb], bi[nb], ov, oi);
      if (EPI == EPI_GROUP) {
        const float om = __shfl_xor(lm[nb], off);
        const float os = __shfl_xor(ls[nb], off);
        lse_merge(lm[nb], ls[nb], om, os);
      }
    }
  }
  __syncthreads();  // H buffers are free: reuse LDS as scratch
  float* sv = (float*)smem;
  int32_t* si = (int32_t*)(sv + kWaves * Bp);
  float* sm = (float*)(si + kWaves * Bp);
  float* ss = sm + kWaves * Bp;
  if (grp == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + l16;
      sv[wave * Bp + b] = bv[nb];
      si[wave * Bp + b] = bi[nb];
      sm[wave * Bp + b] = lm[nb];
      ss[wave * Bp + b] = ls[nb];
    }
  }
  __syncthreads();
  publish_tile<EPI>(p, Bp, sv, si, sm, ss);
  finish_tiles<EPI>(p.B, p.n_tiles, p.ws_val, p.ws_idx, p.ws_m, p.ws_s, p.ticket, p.out_idx, p.out_sum);
}

// ---------------------------------------------------------------------------
// Dot-product streaming kernel for small batches (B <= BD <= 8): the same W
// stream, with bf16 pair dot products on the vector ALU against H rows read
// from LDS (one address per 16-lane group, i.e. broadcast reads).  After the
// k loop the four lane groups are summed (two cross-lane steps); lane (r, g)
// then handles row r for batch rows g, g + 4.
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

template <int BD>
__device__ __forceinline__ float pick(const float (&a)[BD], int idx) {
  float r = a[0];
#pragma unroll
  for (int i = 1; i < BD; ++i) r = (idx == i) ? a[i] : r;
  return r;
}

template <int BD, int MB, int EPI>
__global__ void __launch_bounds__(kThreads) fmms_dot_kernel(const StreamParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NS = (BD + 3) / 4;  // batch slots per lane after the cross-group sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const TileRange tr = tile_range<MB>(p);
  const int nsub = p.nsub, cs = p.cs, nchunk = p.nchunk;
  const int total = tr.rounds * nsub;
  const int bufbytes = BD * p.h_rowstride;

  float bv[NS], lm[NS], ls[NS];
  int32_t bi[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    bv[s] = -INFINITY;
    bi[s] = -1;
    lm[s] = -INFINITY;
    ls[s] = 0.0f;
  }
  float acc[MB][BD];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int b = 0; b < BD; ++b) acc[m][b] = 0.0f;

  u32x4_t hs[kMaxStagePieces];
  u32x4_t wa[MB][8], wb[MB][8];
  int cc = 0;

  auto compute = [&](const u32x4_t (&cur)[MB][8], const unsigned char* hbase, int sbc) {
    const unsigned char* hb = hbase + sbc * 512 + grp * 128;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int b = 0; b < BD; ++b) {
        const u32x4_t hv = *(const u32x4_t*)(hb + b * p.h_rowstride + j * 16);
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m][b] = dot8(cur[m][j], hv, acc[m][b]);
      }
    }
  };

  auto epilogue = [&](int rnd) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int b = 0; b < BD; ++b) {
        acc[m][b] += __shfl_xor(acc[m][b], 16);
        acc[m][b] += __shfl_xor(acc[m][b], 32);
      }
      const int64_t mbg = tr.mb_lo + (int64_t)rnd * (kWaves * MB) + wave * MB + m;
      if (mbg < tr.mb_hi) {
        const int64_t v = mbg * 16 + l16;
        const int64_t gv = p.vocab_offset + v;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int b = grp + 4 * s;
          if (b < p.B && b < BD) {
            const float x = pick<BD>(acc[m], b);
            if (EPI == EPI_STORE) {
              if (v < p.V) p.logits[(int64_t)b * p.ldl + v] = x;
            } else {
              const int64_t grow = (int64_t)p.row_offset + b;
              const Philox4 r =
                  philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)(gv >> 2), (uint32_t)grow, p.step_lo, p.step_hi);
              const uint32_t q = (uint32_t)(gv & 3);
              const uint32_t word = q == 0 ? r.w[0] : q == 1 ? r.w[1] : q == 2 ? r.w[2] : r.w[3];
              bool ok = v < p.V;
              if (ok && p.mask) ok = mask_allows(p.mask + grow * p.ldm, gv);
              const float sc = x * p.inv_t;
              const float pv = ok ? sc + gumbel_from_bits(word) : -INFINITY;
              if (pv > bv[s]) {
                bv[s] = pv;
                bi[s] = (int32_t)gv;
              }
              if (EPI == EPI_GROUP && ok) lse_push(lm[s], ls[s], sc);
            }
          }
        }
      }
#pragma unroll
      for (int b = 0; b < BD; ++b) acc[m][b] = 0.0f;
    }
  };

  auto step = [&](int it, const u32x4_t (&cur)[MB][8], u32x4_t (&nxt)[MB][8]) {
    const int rnd = it / nsub;
    const int sb = it - rnd * nsub;
    const int cidx = sb / cs;
    const int sbc = sb - cidx * cs;
    if (it + 1 < total) load_w<MB>(nxt, p, tr, wave, l16, grp, it + 1);
    const bool chunked = nchunk > 1;
    const bool last_chunk_overall = (rnd == tr.rounds - 1) && (cidx == nchunk - 1);
    if (chunked && sbc == 0 && !last_chunk_overall)
      h_prefetch(hs, p, BD, cidx + 1 < nchunk ? cidx + 1 : 0);
    const int buf = (p.nbuf == 2) ? (cc & 1) : 0;
    compute(cur, smem + buf * bufbytes, sbc);
    if (chunked && (sbc == cs - 1 || sb == nsub - 1)) {
      if (!last_chunk_overall) {
        if (p.nbuf == 2) {
          h_commit(hs, p, BD, smem + ((cc + 1) & 1) * bufbytes);
          __syncthreads();
        } else {
          __syncthreads();
          h_commit(hs, p, BD, smem);
          __syncthreads();
        }
      }
      ++cc;
    }
    if (sb == nsub - 1) epilogue(rnd);
  };

  if (total > 0) {
    if (nchunk == 1) {
      h_stage_all(p, BD, 0, smem);
    } else {
      h_prefetch(hs, p, BD, 0);
      h_commit(hs, p, BD, smem);
    }
    __syncthreads();
    load_w<MB>(wa, p, tr, wave, l16, grp, 0);
    for (int it = 0; it < total; it += 2) {
      step(it, wa, wb);
      if (it + 1 < total) step(it + 1, wb, wa);
    }
  }
  if (EPI == EPI_STORE) return;

  // Reduce over the 16 rows of each lane group.
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int off = 1; off <= 8; off <<= 1) {
      const float ov = __shfl_xor(bv[s], off);
      const int32_t oi = __shfl_xor(bi[s], off);
      merge_best(bv[s], bi[s], ov, oi);
      if (EPI == EPI_GROUP) {
        const float om = __shfl_xor(lm[s], off);
        const float os = __shfl_xor(ls[s], off);
        lse_merge(lm[s], ls[s], om, os);
      }
    }
  }
  __syncthreads();
  float* sv = (float*)smem;
  int32_t* si = (int32_t*)(sv + kWaves * BD);
  float* sm = (float*)(si + kWaves * BD);
  float* ss = sm + kWaves * BD;
  if (l16 == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int b = grp + 4 * s;
      if (b < BD) {
        sv[wave * BD + b] = bv[s];
        si[wave * BD + b] = bi[s];
        sm[wave * BD + b] = lm[s];
        ss[wave * BD + b] = ls[s];
      }
    }
  }
  __syncthreads();
  publish_tile<EPI>(p, BD, sv, si, sm, ss);
  finish_tiles<EPI>(p.B, p.n_tiles, p.ws_val, p.ws_idx, p.ws_m, p.ws_s, p.ticket, p.out_idx, p.out_sum);
}

// ---------------------------------------------------------------------------
// Unfused second pass: sample from fp32 logits stored in HBM.  Tile t covers a
// balanced range of vocab quads; wave w handles rows w, w + 8, ...; each lane
// takes one quad (4 ids, one Philox call) at a time.  Same arithmetic as the
// fused epilogue, so the ids are identical for identical logits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) sample_logits_kernel(const SampleParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int64_t nq = (p.V + 3) / 4;
  const int64_t q_lo = (int64_t)t * nq / p.n_tiles, q_hi = (int64_t)(t + 1) * nq / p.n_tiles;
  for (int b = wave; b < p.B; b += kWaves) {
    float bv = -INFINITY;
    int32_t bi = -1;
    const float* row = p.logits + (int64_t)b * p.ldl;
    for (int64_t q = q_lo + lane; q < q_hi; q += 64) {
      const int64_t v0 = q * 4;
      float x[4];
      if (v0 + 3 < p.V) {
        const f32x4_t v4 = *(const f32x4_t*)(row + v0);
        x[0] = v4[0];
        x[1] = v4[1];
        x[2] = v4[2];
        x[3] = v4[3];
      } else {
        for (int i = 0; i < 4; ++i) x[i] = (v0 + i < p.V) ? row[v0 + i] : 0.0f;
      }
      const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)q, (uint32_t)b, p.step_lo, p.step_hi);
      uint32_t bits = 0xFu;
      if (p.mask) bits = (p.mask[(int64_t)b * p.ldm + (v0 >> 5)] >> (uint32_t)(v0 & 31)) & 0xFu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (v0 + i < p.V) && ((bits >> i) & 1u);
        const float pv = ok ? x[i] * p.inv_t + gumbel_from_bits(r.w[i]) : -INFINITY;
        if (pv > bv) {
          bv = pv;
          bi = (int32_t)(v0 + i);
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int32_t oi = __shfl_xor(bi, off);
      merge_best(bv, bi, ov, oi);
    }
    if (lane == 0) {
      p.ws_val[(int64_t)b * p.n_tiles + t] = bv;
      p.ws_idx[(int64_t)b * p.n_tiles + t] = bi;
    }
  }
  finish_tiles<EPI_FLAT>(p.B, p.n_tiles, p.ws_val, p.ws_idx, nullptr, nullptr, p.ticket, p.out_idx, nullptr);
}

// ---------------------------------------------------------------------------
// Grouped combine: one thread per row.
// ---------------------------------------------------------------------------
__global__ void group_combine_kernel(const GroupSummary* __restrict__ s, int n_groups, int B, uint32_t seed_lo,
                                     uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi, int mode,
                                     int32_t* __restrict__ out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  float best = -INFINITY;
  int kbest = -1;
  for (int k = 0; k < n_groups; ++k) {
    const GroupSummary g = s[(int64_t)k * B + b];
    float key;
    if (mode == 0) {
      const Philox4 r = philox4x32_10(seed_lo, seed_hi, 0x40000000u | (uint32_t)k, (uint32_t)b, step_lo, step_hi);
      key = g.lse + gumbel_from_bits(r.w[0]);
    } else {
      key = g.pmax;
    }
    if (key > best) {
      best = key;
      kbest = k;
    }
  }
  out[b] = kbest < 0 ? -1 : s[(int64_t)kbest * B + b].arg;
}

// ---------------------------------------------------------------------------
// Test exports.
// ---------------------------------------------------------------------------
__global__ void debug_philox_kernel(uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi,
                                    uint32_t row, int64_t v0, int64_t n, uint32_t* r_out, float* g_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t v = v0 + i;
  const Philox4 r = philox4x32_10(seed_lo, seed_hi, (uint32_t)(v >> 2), row, step_lo, step_hi);
  const uint32_t q = (uint32_t)(v & 3);
  const uint32_t w = q == 0 ? r.w[0] : q == 1 ? r.w[1] : q == 2 ? r.w[2] : r.w[3];
  if (r_out) r_out[i] = w;
  if (g_out) g_out[i] = gumbel_from_bits(w);
}

__global__ void debug_gumbel_bits_kernel(uint64_t r0, int64_t n, float* g_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  g_out[i] = gumbel_from_bits((uint32_t)(r0 + (uint64_t)i));
}

__device__ __forceinline__ uint32_t order_key(float f) {  // monotone map float -> uint32
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 2^20 threads, 4096 consecutive words each.  stats: [0] nonfinite, [1]
// decreases, [2] min key, [3] max key (converted to float bits afterwards).
__global__ void debug_gumbel_scan_kernel(unsigned long long* stats) {
  const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t r_lo = t * 4096u, r_hi = r_lo + 4096u;
  unsigned long long nonfinite = 0, decreases = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  float prev = r_lo > 0 ? gumbel_from_bits((uint32_t)(r_lo - 1)) : -INFINITY;
  for (uint64_t r = r_lo; r < r_hi; ++r) {
    const float g = gumbel_from_bits((uint32_t)r);
    nonfinite += !isfinite(g);
    decreases += (g < prev);
    const uint32_t k = order_key(g);
    kmin = k < kmin ? k : kmin;
    kmax = k > kmax ? k : kmax;
    prev = g;
  }
  // wave-level combine, then one atomic per wave
  for (int off = 32; off >= 1; off >>= 1) {
    nonfinite += __shfl_xor(nonfinite, off);
    decreases += __shfl_xor(decreases, off);
    const uint32_t a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&stats[0], nonfinite);
    atomicAdd(&stats[1], decreases);
    atomicMin(&stats[2], (unsigned long long)kmin);
    atomicMax(&stats[3], (unsigned long long)kmax);
  }
}

__global__ void debug_gumbel_scan_finish(unsigned long long* stats) {
  stats[2] = (unsigned long long)__float_as_uint(order_key_inv((uint32_t)stats[2]));
  stats[3] = (unsigned long long)__float_as_uint(order_key_inv((uint32_t)stats[3]));
}

__global__ void debug_gumbel_scan_init(unsigned long long* stats) {
  stats[0] = 0;
  stats[1] = 0;
  stats[2] = 0xFFFFFFFFull;
  stats[3] = 0;
}

// ---------------------------------------------------------------------------
// Host side: planning and launches.
// ---------------------------------------------------------------------------
bool plan_stream(StreamParams& p, StreamConfig& cfg) {
  const int Bp = cfg.dot ? cfg.bd : cfg.nb * 16;
  p.nsub = (p.d + 255) / 256;
  const int scratch = kWaves * Bp * 16;
  auto rowstride = [](int cs) { return cs * 512 + 16; };
  if ((int64_t)Bp * rowstride(p.nsub) <= kLdsMax) {  // whole H resident
    p.cs = p.nsub;
    p.nchunk = 1;
    p.nbuf = 1;
  } else {
    int cs = 0;
    for (int c = p.nsub; c >= 1; --c) {
      if ((int64_t)2 * Bp * rowstride(c) <= kLdsMax && Bp * c * 32 <= kMaxStagePieces * kThreads) {
        cs = c;
        break;
      }
    }
    if (cs > 0) {
      p.cs = cs;
      p.nbuf = 2;
    } else if ((int64_t)Bp * rowstride(1) <= kLdsMax && Bp * 32 <= kMaxStagePieces * kThreads) {
      p.cs = 1;
      p.nbuf = 1;
    } else {
      return false;
    }
    p.nchunk = (p.nsub + p.cs - 1) / p.cs;
    if (p.nchunk == 1) p.nbuf = 1;
  }
  p.h_rowstride = rowstride(p.cs);
  const int hbytes = p.nbuf * Bp * p.h_rowstride;
  cfg.lds_bytes = hbytes > scratch ? hbytes : scratch;
  return true;
}

template <typename K>
static hipError_t launch_with_lds(K kernel, int grid, int lds, hipStream_t stream, const StreamParams& p) {
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_stream_epi(const StreamParams& p, const StreamConfig& c, hipStream_t s) {
  const int g = p.n_tiles, L = c.lds_bytes;
  if (c.dot) {
    switch (c.bd) {
      case 1: return launch_with_lds(fmms_dot_kernel<1, 1, EPI>, g, L, s, p);
      case 2: return launch_with_lds(fmms_dot_kernel<2, 1, EPI>, g, L, s, p);
      case 4: return launch_with_lds(fmms_dot_kernel<4, 1, EPI>, g, L, s, p);
      case 8: return launch_with_lds(fmms_dot_kernel<8, 1, EPI>, g, L, s, p);
      default: return hipErrorInvalidValue;
    }
  }
  if (c.mb == 1) {
    switch (c.nb) {
      case 1: return launch_with_lds(fmms_mfma_kernel<1, 1, EPI>, g, L, s, p);
      case 2: return launch_with_lds(fmms_mfma_kernel<2, 1, EPI>, g, L, s, p);
      case 4: return launch_with_lds(fmms_mfma_kernel<4, 1, EPI>, g, L, s, p);
      default: return hipErrorInvalidValue;
    }
  }
  switch (c.nb) {
    case 1: return launch_with_lds(fmms_mfma_kernel<1, 2, EPI>, g, L, s, p);
    case 2: return launch_with_lds(fmms_mfma_kernel<2, 2, EPI>, g, L, s, p);
    case 4: return launch_with_lds(fmms_mfma_kernel<4, 2, EPI>, g, L, s, p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream(const StreamParams& p, const StreamConfig& cfg, int epi, hipStream_t stream) {
  switch (epi) {
    case EPI_FLAT: return launch_stream_epi<EPI_FLAT>(p, cfg, stream);
    case EPI_GROUP: return launch_stream_epi<EPI_GROUP>(p, cfg, stream);
    case EPI_STORE: return launch_stream_epi<EPI_STORE>(p, cfg, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sample_logits(const SampleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(sample_logits_kernel, dim3(p.n_tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_group_combine(const GroupSummary* s, int n_groups, int B, uint64_t seed, uint64_t step, int mode,
                                int32_t* out_idx, hipStream_t stream) {
  const int threads = 256;
  hipLaunchKernelGGL(group_combine_kernel, dim3((B + threads - 1) / threads), dim3(threads), 0, stream, s, n_groups,
                     B, (uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)step, (uint32_t)(step >> 32), mode, out_idx);
  return hipGetLastError();
}

hipError_t launch_debug_philox(uint64_t seed, uint64_t step, uint32_t row, int64_t v0, int64_t n, uint32_t* r_out,
                               float* g_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(debug_philox_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, (uint32_t)seed,
                     (uint32_t)(seed >> 32), (uint32_t)step, (uint32_t)(step >> 32), row, v0, n, r_out, g_out);
  return hipGetLastError();
}

hipError_t launch_debug_gumbel_bits(uint64_t r0, int64_t n, float* g_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(debug_gumbel_bits_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, r0, n, g_out);
  return hipGetLastError();
}

hipError_t launch_debug_gumbel_scan(unsigned long long* stats, hipStream_t stream) {
  hipLaunchKernelGGL(debug_gumbel_scan_init, dim3(1), dim3(1), 0, stream, stats);
  // 4096 blocks x 256 threads x 4096 words = 2^32 words
  hipLaunchKernelGGL(debug_gumbel_scan_kernel, dim3(4096), dim3(256), 0, stream, stats);
  hipLaunchKernelGGL(debug_gumbel_scan_finish, dim3(1), dim3(1), 0, stream, stats);
  return hipGetLastError();
}

}  // namespace fsk
