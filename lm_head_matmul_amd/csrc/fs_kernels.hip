// fs_kernels.hip -- the FlashSampling kernels around the streaming pass on
// MI355X (gfx950): the unfused comparator's sampling pass, the grouped
// combine, test exports, and host-side planning / dispatch of all launches.
#include "fs_stream.h"

namespace fsk {

// The streaming launches are instantiated in fs_stream_{flat,group,store,topk}.hip.
extern template hipError_t launch_stream_epi<EPI_FLAT>(const StreamParams&, const StreamConfig&, hipStream_t);
extern template hipError_t launch_stream_epi<EPI_GROUP>(const StreamParams&, const StreamConfig&, hipStream_t);
extern template hipError_t launch_stream_epi<EPI_STORE>(const StreamParams&, const StreamConfig&, hipStream_t);
extern template hipError_t launch_stream_epi<EPI_TOPK>(const StreamParams&, const StreamConfig&, hipStream_t);

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
    wave_best(bv, bi);
    if (lane == 0) {
      p.ws_val[(int64_t)b * p.n_tiles + t] = bv;
      p.ws_idx[(int64_t)b * p.n_tiles + t] = bi;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k sampling from stored logits: exact top-k of the allowed scores
// s = logit * (1/T), ties at the boundary kept by lower id, then the
// Gumbel-max over the kept ids.  [readus.org FlashSampling summary, section on
// Top-K and masking: the sampler acts on the kept set]
//
// Keys are order-preserving 32-bit images of the scores; the boundary is found
// by a most-significant-digit radix select whose first level histograms key
// bits 31..20.  Two launches per batch chunk, each row split into segments:
//   1. histogram: every (segment, row) workgroup counts its keys in LDS, finds
//      its own boundary bin (where its count from the top reaches k) and adds
//      its non-zero bins from there up into the row's histogram in global
//      memory.  The row's last workgroup to arrive (a per-row arrival counter)
//      reads the histogram back, stores the row's boundary -- the bin where the
//      count from the top reaches k, the count above that bin, the count inside
//      it and the total -- and leaves the histogram and the counter at zero for
//      the next call;
//   2. collect: every (segment, row) workgroup takes the Gumbel-max over its
//      ids above the boundary bin and appends its ids inside the bin to the
//      row's candidate list.  The row's last workgroup to arrive ranks the
//      candidates by (key desc, id asc), perturbs the first k - above of them,
//      merges them with the segments' maximizers, writes the sample and leaves
//      the candidate count and the counter at zero.
// What one workgroup hands to a row's last one goes through device-scope
// atomics (histogram adds, candidate and maximizer stores, their loads), which
// are coherent across the chip's L2 caches; every thread waits for its own to
// complete before the workgroup counts its arrival.  A device-scope fence would
// do the same by writing back and invalidating whole L2 caches, which costs
// far more than the pass.
// A boundary bin holding more than kTopkCap ids (very narrow score ranges) is
// resolved by the last collect workgroup alone: it refines the bin on key bits
// 19..8 and 7..0 and, if more than kTopkCap ids share the exact boundary key,
// keeps the lowest of them by a pass in id order.
// ---------------------------------------------------------------------------
// Order-preserving key of a score, with -0 folded onto +0 (they compare equal).
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Device-scope loads and stores of the words workgroups hand to each other.
template <class T>
__device__ __forceinline__ void dev_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T dev_load(T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static_assert(kTopkCap * 8 == kTopkBins * 4, "candidate list and refinement histogram share LDS");
static_assert(kTopkBins % kThreads == 0, "whole runs of bins per thread");

struct TopkShared {
  union {
    uint32_t hist[kTopkBins];  // refinement levels of a row resolved alone
    uint64_t cand[kTopkCap];   // boundary candidates (key << 32 | ~id)
  };
  int bin, above, inbin, total, ncand, run, last;
  float red_v[kWaves];
  int32_t red_i[kWaves];
};

// Wave 0: the boundary of an LDS histogram of nbins bins (counts from the top):
// total count, the bin where the running count from the top reaches `need`,
// the count above that bin and the count inside it.  If total < need the bin
// fields are left unset.
__device__ __forceinline__ void topk_boundary(const uint32_t* h, int nbins, int need, TopkShared& sh) {
  const int lane = threadIdx.x & 63;
  const int per = nbins / 64;  // lane l owns bins [hi - (l + 1) * per, hi - l * per) counted from the top
  const int top = nbins - 1 - lane * per;
  int local = 0;
  for (int j = 0; j < per; ++j) local += (int)h[top - j];
  int incl = local;  // inclusive prefix over lanes 0..lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - local;
  const int total = __shfl(incl, 63);
  if (lane == 0) sh.total = total;
  if (excl < need && incl >= need) {
    int run = excl;
    for (int j = 0; j < per; ++j) {
      const int c = (int)h[top - j];
      if (run + c >= need) {
        sh.bin = top - j;
        sh.above = run;
        sh.inbin = c;
        break;
      }
      run += c;
    }
  }
}

constexpr int kTopkPer = kTopkBins / kThreads;  // histogram bins per thread in the block-wide scans

// The whole workgroup: boundary of a histogram whose bins are held kTopkPer to
// a thread (thread t holds c[0..kTopkPer) of bins base .. base + kTopkPer - 1,
// the ones that come t-th from the top), written as {bin, above, inbin, total}
// to out ({-1, 0, 0, total} when total < need).  out is read after the
// caller's next barrier; wsum is LDS scratch of kWaves words.
__device__ __forceinline__ void topk_boundary_block(const uint32_t (&c)[kTopkPer], int base, int need, int32_t* wsum,
                                                    int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int local = 0;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) local += (int)c[j];
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = wsum[w];
    if (w < wave) incl += s;
    total += s;
  }
  const int excl = incl - local;
  if (tid == 0) {
    out[3] = total;
    if (total < need) {
      out[0] = -1;
      out[1] = 0;
      out[2] = 0;
    }
  }
  if (excl < need && incl >= need) {
    int run = excl;
#pragma unroll
    for (int j = kTopkPer - 1; j >= 0; --j) {
      const int n = (int)c[j];
      if (run < need && run + n >= need) {
        out[0] = base + j;
        out[1] = run;
        out[2] = n;
      }
      run += n;
    }
  }
}

// Workgroup maximizer; the result is valid in thread 0.
__device__ __forceinline__ void topk_block_best(float& bv, int32_t& bi, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_best(bv, bi);
  __syncthreads();
  if (lane == 0) {
    sh.red_v[wave] = bv;
    sh.red_i[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 0; w < kWaves; ++w) merge_best(bv, bi, sh.red_v[w], sh.red_i[w]);
}

// Arrival of a workgroup at a per-row counter once its device-scope writes
// have completed; true in every thread of the row's last workgroup, which may
// then read them with device-scope loads.  The last one resets the counter.
__device__ __forceinline__ bool topk_arrive_last(uint32_t* counter, int n, int& flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's atomics and stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool last = atomicAdd(counter, 1u) == (uint32_t)(n - 1);
    if (last) dev_store(counter, 0u);
    flag = last;
  }
  __syncthreads();
  return flag != 0;
}

// Row view shared by the launches.
struct TopkRow {
  const float* L;
  const uint32_t* M;
  uint32_t grow;
  int V;
  float inv_t;
  __device__ bool allowed(int v) const { return M == nullptr || ((M[v >> 5] >> (v & 31)) & 1u); }
  __device__ float score(int v) const { return L[v] * inv_t; }
};

__device__ __forceinline__ TopkRow topk_row(const TopkParams& p, int b) {
  TopkRow r;
  r.L = p.logits + (int64_t)b * p.ldl;
  r.grow = (uint32_t)(p.row_offset + b);
  r.M = p.mask ? p.mask + (int64_t)r.grow * p.ldm : nullptr;
  r.V = p.V;
  r.inv_t = p.inv_t;
  return r;
}

// Perturb a kept id and update the maximizer.
__device__ __forceinline__ void topk_take(const TopkParams& p, const TopkRow& row, int v, float s, float& bv,
                                          int32_t& bi) {
  const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)v >> 2, row.grow, p.step_lo, p.step_hi);
  const uint32_t q = (uint32_t)v & 3u;
  const uint32_t w = q == 0 ? r.w[0] : q == 1 ? r.w[1] : q == 2 ? r.w[2] : r.w[3];
  merge_best(bv, bi, s + gumbel_from_bits(w), v);
}

// Visits the allowed ids of quads [q_lo, q_hi) of a row, four quads per
// thread in flight: f(v, s, key).
template <class F>
__device__ __forceinline__ void topk_scan(const TopkRow& row, int64_t q_lo, int64_t q_hi, F&& f) {
  constexpr int U = 4;
  for (int64_t q0 = q_lo + threadIdx.x; q0 < q_hi; q0 += U * kThreads) {
    f32x4_t x[U];
    uint32_t bits[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + (int64_t)u * kThreads;
      bits[u] = 0;
      if (q < q_hi) {
        const int v0 = (int)(q * 4);
        x[u] = *(const f32x4_t*)(row.L + v0);  // rows are padded to whole quads
        bits[u] = row.M ? (row.M[v0 >> 5] >> (uint32_t)(v0 & 31)) & 0xFu : 0xFu;
        const int left = row.V - v0;
        if (left < 4) bits[u] &= (1u << left) - 1u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v0 = (int)((q0 + (int64_t)u * kThreads) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((bits[u] >> i) & 1u) {
          const float s = x[u][i] * row.inv_t;
          f(v0 + i, s, score_key(s));
        }
    }
  }
}

__device__ __forceinline__ void topk_segment(const TopkParams& p, int seg, int64_t& q_lo, int64_t& q_hi) {
  const int64_t nq = (p.V + 3) / 4;
  q_lo = (int64_t)seg * nq / p.n_seg;
  q_hi = (int64_t)(seg + 1) * nq / p.n_seg;
}

__global__ void __launch_bounds__(kThreads) topk_hist_kernel(const TopkParams p) {
  __shared__ uint32_t hist[kTopkBins];
  __shared__ int32_t wsum[kWaves];
  __shared__ int32_t local_bound[4];
  __shared__ int last;
  const int seg = blockIdx.x, b = blockIdx.y;
  const TopkRow row = topk_row(p, b);
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  int64_t q_lo, q_hi;
  topk_segment(p, seg, q_lo, q_hi);
  topk_scan(row, q_lo, q_hi, [&](int, float, uint32_t key) { atomicAdd(&hist[key >> 20], 1u); });
  __syncthreads();
  // Only the bins from this segment's own boundary up are added to the row's
  // histogram: the row's boundary is never below a segment's (that segment
  // alone has k ids from its boundary up), so every bin from the row's
  // boundary up gets all its counts.  The row's total is exact when it is
  // below k (no segment is cut then).
  const int base = kTopkBins - kTopkPer * ((int)threadIdx.x + 1);
  uint32_t c[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) c[j] = hist[base + j];
  topk_boundary_block(c, base, p.top_k, wsum, local_bound);
  __syncthreads();
  const int floor_bin = local_bound[0] < 0 ? 0 : local_bound[0];
  uint32_t* gh = p.hist + (int64_t)b * kTopkBins;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j)
    if (base + j >= floor_bin && c[j]) atomicAdd(&gh[base + j], c[j]);
  if (!topk_arrive_last(p.arrive_hist + b, p.n_seg, last)) return;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) c[j] = dev_load(gh + base + j);
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) dev_store(gh + base + j, 0u);
  topk_boundary_block(c, base, p.top_k, wsum, p.bound + 4 * (int64_t)b);
}

// Sorts sh.cand[0, n) descending (bitonic, padded with zeros to a power of 2).
__device__ __forceinline__ void topk_sort_desc(TopkShared& sh, int n) {
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  for (int i = n + (int)threadIdx.x; i < np2; i += kThreads) sh.cand[i] = 0;
  __syncthreads();
  for (int kk = 2; kk <= np2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < np2; i += kThreads) {
        const int ij = i ^ j;
        if (ij > i) {
          const uint64_t x = sh.cand[i], y = sh.cand[ij];
          const bool desc = (i & kk) == 0;
          if (desc ? (x < y) : (x > y)) {
            sh.cand[i] = y;
            sh.cand[ij] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int cand_id(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFu)); }

// The whole selection for one row by one workgroup (boundary bins wider than
// kTopkCap): the maximizer over the kept ids, valid in every thread's (bv, bi)
// after the caller's block reduction.
__device__ void topk_row_alone(const TopkParams& p, const TopkRow& row, TopkShared& sh, float& bv, int32_t& bi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = row.V;
  uint32_t prefix = 0, pmask = 0;
  int need = p.top_k;
  int shift = 20, nbins = kTopkBins;
  int level = 0;
  for (; level < 3; ++level) {
    for (int i = tid; i < nbins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int v = tid; v < V; v += kThreads) {
      if (!row.allowed(v)) continue;
      const uint32_t k = score_key(row.score(v));
      if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    if (wave == 0) topk_boundary(sh.hist, nbins, need, sh);
    __syncthreads();
    need -= sh.above;
    prefix |= (uint32_t)sh.bin << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    if (sh.inbin <= kTopkCap) break;
    if (level == 0) {
      shift = 8;
      nbins = 4096;
    } else {
      shift = 0;
      nbins = 256;
    }
    __syncthreads();  // the boundary fields are rewritten by the next level
  }
  if (level < 3) {
    // kept ids above the boundary; boundary candidates into LDS, sorted
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    for (int v = tid; v < V; v += kThreads) {
      if (!row.allowed(v)) continue;
      const float s = row.score(v);
      const uint32_t k = score_key(s);
      const uint32_t hi = k & pmask;
      if (hi > prefix) {
        topk_take(p, row, v, s, bv, bi);
      } else if (hi == prefix) {
        const int at = atomicAdd(&sh.ncand, 1);
        sh.cand[at] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
      }
    }
    __syncthreads();
    const int n = sh.ncand;
    topk_sort_desc(sh, n);
    for (int i = tid; i < need && i < n; i += kThreads) {
      const int v = cand_id(sh.cand[i]);
      topk_take(p, row, v, row.score(v), bv, bi);
    }
  } else {
    // more than kTopkCap ids share the exact boundary key: keys above it are
    // kept, and of those equal to it the `need` lowest ids, found in id order
    if (tid == 0) sh.run = 0;
    __syncthreads();
    for (int base = 0; base < V; base += kThreads) {
      const int v = base + tid;
      bool eq = false;
      if (v < V && row.allowed(v)) {
        const float s = row.score(v);
        const uint32_t k = score_key(s);
        if (k > prefix) topk_take(p, row, v, s, bv, bi);
        eq = k == prefix;
      }
      const uint64_t bal = __ballot(eq);
      const int before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) sh.red_i[wave] = __popcll(bal);
      __syncthreads();
      int before = sh.run;
      for (int w = 0; w < wave; ++w) before += sh.red_i[w];
      if (eq && before + before_in_wave < need) topk_take(p, row, v, row.score(v), bv, bi);
      __syncthreads();
      if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < kWaves; ++w) tot += sh.red_i[w];
        sh.run += tot;
      }
      __syncthreads();
    }
  }
}

// The last collect workgroup of a row: merges the segments' maximizers with
// the perturbed first `need` boundary candidates and writes the row's sample.
__device__ void topk_finish_row(const TopkParams& p, const TopkRow& row, int b, bool keep_all, int above, int inbin,
                                TopkShared& sh) {
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int32_t bi = -1;
  if (keep_all || inbin <= kTopkCap) {
    for (int i = tid; i < p.n_seg; i += kThreads)
      merge_best(bv, bi, dev_load(p.seg_val + (int64_t)b * kTopkMaxSeg + i),
                 dev_load(p.seg_idx + (int64_t)b * kTopkMaxSeg + i));
    if (!keep_all) {
      const int need = p.top_k - above;
      uint64_t* cand = p.cand + (int64_t)b * kTopkCap;
      if (inbin <= kThreads) {
        // one candidate per thread, kept if fewer than `need` candidates rank above it
        const uint64_t mine = tid < inbin ? dev_load(cand + tid) : 0ull;
        if (tid < inbin) sh.cand[tid] = mine;
        __syncthreads();
        if (tid < inbin) {
          int rank = 0;
          for (int j = 0; j < inbin; ++j) rank += sh.cand[j] > mine ? 1 : 0;
          if (rank < need) {
            const int v = cand_id(mine);
            topk_take(p, row, v, row.score(v), bv, bi);
          }
        }
      } else {
        for (int i = tid; i < inbin; i += kThreads) sh.cand[i] = dev_load(cand + i);
        topk_sort_desc(sh, inbin);  // begins with a barrier-separated fill
        for (int i = tid; i < need; i += kThreads) {
          const int v = cand_id(sh.cand[i]);
          topk_take(p, row, v, row.score(v), bv, bi);
        }
      }
    }
  } else {
    topk_row_alone(p, row, sh, bv, bi);
  }
  topk_block_best(bv, bi, sh);
  if (tid == 0) {
    p.out_idx[b] = bi;
    dev_store(p.cand_n + b, 0);
  }
}

__global__ void __launch_bounds__(kThreads) topk_collect_kernel(const TopkParams p) {
  __shared__ TopkShared sh;
  const int seg = blockIdx.x, b = blockIdx.y;
  const TopkRow row = topk_row(p, b);
  const int32_t* bd = p.bound + 4 * (int64_t)b;
  const int bnd_bin = bd[0], above = bd[1], inbin = bd[2], total = bd[3];
  const bool keep_all = total < p.top_k;  // the total is exact only then
  const uint32_t bin = keep_all ? 0u : (uint32_t)bnd_bin;
  const bool collect = !keep_all && inbin <= kTopkCap;
  float bv = -INFINITY;
  int32_t bi = -1;
  int64_t q_lo, q_hi;
  topk_segment(p, seg, q_lo, q_hi);
  if (threadIdx.x == 0) sh.ncand = 0;
  __syncthreads();
  // this segment's boundary candidates go to LDS first (at most the bin's count,
  // <= kTopkCap), then to the row's list with one global atomic per workgroup;
  // a row whose bin is wider than that is left to its last workgroup
  if (keep_all || collect)
    topk_scan(row, q_lo, q_hi, [&](int v, float s, uint32_t key) {
      const uint32_t hi = key >> 20;
      if (keep_all || hi > bin) {
        topk_take(p, row, v, s, bv, bi);
      } else if (hi == bin) {
        const int at = atomicAdd(&sh.ncand, 1);
        sh.cand[at] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
      }
    });
  topk_block_best(bv, bi, sh);  // its barriers also publish sh.ncand and sh.cand
  const int n = sh.ncand;
  if (threadIdx.x == 0) {
    dev_store(p.seg_val + (int64_t)b * kTopkMaxSeg + seg, bv);
    dev_store(p.seg_idx + (int64_t)b * kTopkMaxSeg + seg, bi);
    sh.run = n > 0 ? atomicAdd(&p.cand_n[b], n) : 0;
  }
  __syncthreads();
  uint64_t* cand = p.cand + (int64_t)b * kTopkCap + sh.run;
  for (int i = threadIdx.x; i < n; i += kThreads) dev_store(cand + i, sh.cand[i]);
  if (!topk_arrive_last(p.arrive_coll + b, p.n_seg, sh.last)) return;
  topk_finish_row(p, row, b, keep_all, above, inbin, sh);
}
// ---------------------------------------------------------------------------
// Fused top-k, second launch: one workgroup per batch row merges the lists the
// streaming pass (EPI_TOPK) left per tile: kTopkLane keys and a bound on the
// keys that tile dropped.  [readus.org FlashSampling summary, section on
// Top-K and masking: a pre-filter keeps candidates, exact Gumbel-Max runs on
// them]  Keys order (score desc, id asc); the row's top-k is the k largest.
//   1. theta, a lower bound of the row's k-th key tau: each wave takes the
//      ceil(k/4)-th largest score word of its 64 tiles' maxima (a ballot
//      select); the smallest of the four leaves at least k tile maxima, i.e. k
//      distinct ids, at or above it.  Only list entries >= theta can be kept:
//      they are gathered.  Without such a bound, or if it gathers more than
//      32 k entries, theta is the k-th largest tile maximum itself (then at
//      most kTopkLane k entries reach it).
//   2. tau = the k-th largest gathered key (0 = keep all if there are fewer).
//   3. A tile whose bound reaches tau may have dropped a kept id.  Then the
//      tile is rescored (every id of the tile recomputed from H and W in fp32)
//      and the selection redone over the other tiles' lists and the rescored
//      ids, with the threshold lowered by the near-tie margin so that another
//      fp32 summation order cannot push one of the k tile maxima under it;
//      repeated until no unrescored tile's bound reaches tau.  On the decode
//      workloads no bound comes near tau; ties and tiny vocabularies take it.
//   4. Gumbel-max over the kept ids with the per-id noise of the plain sampler.
// Thread t holds tile t's list (n_tiles <= kTopkMergeThreads).
// ---------------------------------------------------------------------------
static_assert(kTopkMergeThreads == 256 && kTopkMergeCap % kTopkMergeThreads == 0, "merge geometry");
// every list entry of every tile fits the gather buffer, so the fallback
// gather (theta = the k-th tile maximum) needs no bound check
static_assert(kTopkLane * kTopkMergeThreads <= kTopkMergeCap, "one list per tile fits the gather buffer");
static_assert(kTopkFusedMax <= 64, "the nucleus cut sorts the kept keys within one wave");

// Wave-wide bitonic sort, descending, of one 64-bit key per lane.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const uint64_t o = __shfl_xor(x, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & kk) == 0);
      x = keep_max ? (x > o ? x : o) : (x < o ? x : o);
    }
  }
  return x;
}

// k-th largest (1-based) of one 32-bit value per lane over the lanes where
// `valid`, by a most-significant-bit-first select with ballots (no shuffles);
// on return *rest is that value's rank among the equal values (1-based).
// 0 if fewer than kth lanes are valid.
__device__ __forceinline__ uint32_t wave_kth_largest_u32(uint32_t v, bool valid, int kth, int* rest) {
  if (__popcll(__ballot(valid)) < kth) {
    *rest = 0;
    return 0u;
  }
  uint32_t prefix = 0, pmask = 0;
  int need = kth;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t m = 1u << bit;
    const int c = __popcll(__ballot(valid && (v & pmask) == prefix && (v & m) != 0));
    if (c >= need)
      prefix |= m;
    else
      need -= c;
    pmask |= m;
  }
  *rest = need;
  return prefix;
}

struct TopkMergeShared {
  alignas(16) uint64_t F[kTopkMergeCap];  // gathered keys
  uint16_t Ft[kTopkMergeCap];  // tile of each gathered key
  alignas(16) uint64_t S[kTopkMergeThreads];
  uint64_t Tw[kTopkMergeThreads / 64];
  int rescored[kTopkMergeThreads];
  int nF, nnew;
  uint64_t theta, tau;
  float red_v[kTopkMergeThreads / 64];
  int32_t red_i[kTopkMergeThreads / 64];
};

// Rank of one key per thread (0: none) among the block's keys: the waves sort
// their keys, then each key's rank is its lane plus, for every other wave, the
// count of that wave's keys above it (binary search).  On return x is the key
// the thread now holds.  Non-zero keys are distinct.
__device__ __forceinline__ int block_rank(uint64_t& x, TopkMergeShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sort_desc(x);
  sh.S[threadIdx.x] = x;
  __syncthreads();
  int r = lane;
  for (int w = 0; w < kTopkMergeThreads / 64; ++w) {
    if (w == wave) continue;
    const uint64_t* L = sh.S + w * 64;
    int lo = 0, hi = 64;  // first entry of the descending list L that is not above x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L[mid] > x)
        lo = mid + 1;
      else
        hi = mid;
    }
    r += lo;
  }
  __syncthreads();
  return r;
}

// Count of the n keys of F (LDS, 16-byte aligned) above x: every thread reads
// the same words, 8 keys per batch of loads so that their latency overlaps.
__device__ __forceinline__ int rank_in(const uint64_t* F, int n, uint64_t x) {
  int r = 0, j = 0;
  for (; j + 8 <= n; j += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = F[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += v[u] > x ? 1 : 0;
  }
  for (; j < n; ++j) r += F[j] > x ? 1 : 0;
  return r;
}

// The k-th largest of the gathered keys, 0 if there are fewer than k.
__device__ uint64_t topk_select_kth(TopkMergeShared& sh, int k) {
  __syncthreads();
  const int n = sh.nF;
  if (threadIdx.x == 0) sh.tau = 0;
  if (n <= kTopkMergeThreads) {
    uint64_t x = (int)threadIdx.x < n ? sh.F[threadIdx.x] : 0ull;
    const int r = block_rank(x, sh);  // its first barrier orders the store to tau above
    if (x != 0 && r == k - 1) sh.tau = x;
  } else {
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kTopkMergeThreads) {
      const uint64_t x = sh.F[i];
      if (rank_in(sh.F, n, x) == k - 1) sh.tau = x;
    }
  }
  __syncthreads();
  return sh.tau;
}

// Keeps the k largest gathered keys (moved to the front).
__device__ __noinline__ void topk_compact(TopkMergeShared& sh, int k) {
  constexpr int kPer = kTopkMergeCap / kTopkMergeThreads;
  __syncthreads();
  const int n = sh.nF;
  uint64_t key[kPer];
  int rank[kPer];
  uint16_t tile[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = threadIdx.x + q * kTopkMergeThreads;
    key[q] = i < n ? sh.F[i] : 0ull;
    tile[q] = i < n ? sh.Ft[i] : (uint16_t)0;
    rank[q] = key[q] != 0 ? rank_in(sh.F, n, key[q]) : INT32_MAX;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPer; ++q)
    if (rank[q] < k) {
      sh.F[rank[q]] = key[q];
      sh.Ft[rank[q]] = tile[q];
    }
  __syncthreads();
  if (threadIdx.x == 0) sh.nF = n < k ? n : k;
  __syncthreads();
}

// Block-wide append of one key per thread (0: none); compacts first when a
// full round might not fit.  Every thread of the block calls it.
__device__ __forceinline__ void topk_append(TopkMergeShared& sh, uint64_t key, int tile, int k) {
  __syncthreads();
  if (sh.nF + kTopkMergeThreads > kTopkMergeCap) topk_compact(sh, k);
  if (key != 0) {
    const int i = atomicAdd(&sh.nF, 1);
    sh.F[i] = key;
    sh.Ft[i] = (uint16_t)tile;
  }
}

// Score of vocab row v (local to the launch) for batch row b, recomputed in fp32.
__device__ float topk_rescore(const StreamParams& p, int b, int v) {
  const uint16_t* h = p.H + (int64_t)b * p.ldh;
  const uint16_t* w = p.W + (int64_t)v * p.ldw;
  float acc = 0.0f;
  for (int k = 0; k < p.d; k += 8) {
    const u32x4_t hv = *(const u32x4_t*)(h + k);
    const u32x4_t wv = *(const u32x4_t*)(w + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(__uint_as_float(hv[i] << 16), __uint_as_float(wv[i] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(hv[i] & 0xFFFF0000u), __uint_as_float(wv[i] & 0xFFFF0000u), acc);
    }
  }
  return acc * p.inv_t;
}

__global__ void __launch_bounds__(kTopkMergeThreads) topk_merge_kernel(const StreamParams p) {
  __shared__ TopkMergeShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  const int nt = p.n_tiles, k = p.top_k;
  const bool has = tid < nt;
  const uint64_t* cand = p.topk_cand + (int64_t)b * kTopkSlot * nt;
  const uint32_t row = (uint32_t)(p.row_offset + b);
  auto noise_of = [&](int32_t id) {
    const Philox4 rr = philox4x32_10(p.seed_lo, p.seed_hi, (uint32_t)id >> 2, row, p.step_lo, p.step_hi);
    const uint32_t q = (uint32_t)id & 3u;
    return gumbel_from_bits(q == 0 ? rr.w[0] : q == 1 ? rr.w[1] : q == 2 ? rr.w[2] : rr.w[3]);
  };
  // this thread's tile: its kTopkLane best keys (descending) and its bound
  uint64_t e[kTopkLane];
#pragma unroll
  for (int j = 0; j < kTopkLane; ++j) e[j] = has ? cand[(int64_t)j * nt + tid] : 0ull;
  const uint64_t hb = has ? cand[(int64_t)kTopkLane * nt + tid] : 0ull;
  // 1. theta, a lower bound of the row's k-th key: in each wave the
  // ceil(k/4)-th largest score among its 64 tile maxima; at least k keys reach
  // the smallest of the four, so every key with at least that score is gathered.
  // If a wave holds fewer keys, or the bound gathers more than 32 k entries,
  // theta is the k-th largest tile maximum itself (ranks by counting over LDS).
  const uint64_t x = e[0];
  sh.S[tid] = x;
  sh.rescored[tid] = 0;
  if (tid == 0) {
    sh.theta = 0;
    sh.tau = 0;
    sh.nF = 0;
    sh.nnew = 0;
  }
  {
    int rest = 0;
    const int kw = (k + kTopkMergeThreads / 64 - 1) / (kTopkMergeThreads / 64);
    const uint32_t t = wave_kth_largest_u32((uint32_t)(x >> 32), x != 0, kw, &rest);
    if (lane == 0) sh.Tw[wave] = t;
  }
  __syncthreads();
  uint32_t t32 = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kTopkMergeThreads / 64; ++w) t32 = (uint32_t)sh.Tw[w] < t32 ? (uint32_t)sh.Tw[w] : t32;
  uint64_t th = (uint64_t)t32 << 32, theta = th;
  int cnt = 0;
  if (t32 != 0) {
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j) cnt += e[j] >= th ? 1 : 0;
    int at = cnt > 0 ? atomicAdd(&sh.nF, cnt) : 0;
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j)
      if (e[j] >= th) {
        if (at < kTopkMergeCap) {
          sh.F[at] = e[j];
          sh.Ft[at] = (uint16_t)tid;
        }
        ++at;
      }
  }
  __syncthreads();
  if (t32 == 0 || sh.nF > 32 * k) {
    if (x != 0 && rank_in(sh.S, nt, x) == k - 1) sh.theta = x;
    __syncthreads();
    theta = sh.theta;
    th = theta != 0 ? theta : 1ull;  // fewer than k tiles hold a key: gather them all
    if (tid == 0) sh.nF = 0;
    __syncthreads();
    cnt = 0;
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j) cnt += e[j] >= th ? 1 : 0;
    int at = cnt > 0 ? atomicAdd(&sh.nF, cnt) : 0;
#pragma unroll
    for (int j = 0; j < kTopkLane; ++j)
      if (e[j] >= th) {
        sh.F[at] = e[j];
        sh.Ft[at] = (uint16_t)tid;
        ++at;
      }
    __syncthreads();
  }
  // 2. tau: the k-th largest gathered key (0 if fewer than k), by ranks
  const int n0 = sh.nF;
  for (int i = tid; i < n0; i += kTopkMergeThreads)
    if (rank_in(sh.F, n0, sh.F[i]) == k - 1) sh.tau = sh.F[i];
  // 3. a tile whose dropped keys could reach tau is rescored
  __syncthreads();
  uint64_t tau = sh.tau;
  bool flag = has && hb != 0 && hb >= tau;
  if (flag) {
    sh.rescored[tid] = 1;
    atomicAdd(&sh.nnew, 1);
  }
  __syncthreads();
  if (sh.nnew != 0) {
    // rebuild: the lists of the other tiles, every id of the rescored ones;
    // repeated while the new tau brings more tiles in
    const uint64_t th2 =
        theta != 0 ? (uint64_t)order_bits(topk_key_score(theta) - 1e-3f * (1.0f + fabsf(topk_key_score(theta)))) << 32
                   : 1ull;
    for (;;) {
      __syncthreads();
      if (tid == 0) sh.nF = 0;
      const bool mine = has && !sh.rescored[tid];
#pragma unroll
      for (int j = 0; j < kTopkLane; ++j) {
        const uint64_t v = mine ? e[j] : 0ull;
        topk_append(sh, v >= th2 ? v : 0ull, tid, k);
      }
#pragma unroll 1
      for (int t = 0; t < nt; ++t) {
        if (!sh.rescored[t]) continue;  // uniform: written before the last barrier
        const int64_t lo = tile_lo(t, p.n_mblocks, p.n_tiles, p.tile_ratio) * 16;
        int64_t hi = tile_lo(t + 1, p.n_mblocks, p.n_tiles, p.tile_ratio) * 16;
        hi = hi < p.V ? hi : p.V;
        const uint32_t* mrow = p.mask ? p.mask + (int64_t)(p.row_offset + b) * p.ldm : nullptr;
#pragma unroll 1
        for (int64_t v0 = lo; v0 < hi; v0 += kTopkMergeThreads) {
          const int64_t v = v0 + tid;
          uint64_t key = 0;
          if (v < hi) {
            const int gv = (int)(p.vocab_offset + v);
            if (mrow == nullptr || mask_allows(mrow, gv)) {
              const float sc = topk_rescore(p, b, (int)v);
              if (sc == sc) key = topk_key(sc, gv);
            }
          }
          topk_append(sh, key >= th2 ? key : 0ull, t, k);
        }
      }
      tau = topk_select_kth(sh, k);
      if (tid == 0) sh.nnew = 0;
      __syncthreads();
      flag = has && !sh.rescored[tid] && hb != 0 && hb >= tau;
      if (flag) {
        sh.rescored[tid] = 1;
        atomicAdd(&sh.nnew, 1);
      }
      __syncthreads();
      if (sh.nnew == 0) break;
    }
  }
  // 4. Gumbel-max over the kept keys (>= tau): all of them, or with top_p < 1
  // the nucleus of the kept ids -- sorted by key, an id stays while the fp64
  // weight exp(s - s_max) of the ids before it is below top_p times their total
  // [nucleus sampling, Holtzman et al., ICLR 2020, over the top-k set]
  const int n = sh.nF;
  float bv = -INFINITY;
  int32_t bi = -1;
  if (p.top_p < 1.0f) {
    // the kept keys (at most k <= 64) in order into S, then wave 0 cuts them
    __syncthreads();
    for (int i = tid; i < n; i += kTopkMergeThreads) {
      const uint64_t key = sh.F[i];
      if (key != 0 && key >= tau) sh.S[rank_in(sh.F, n, key)] = key;
    }
    __syncthreads();
    if (wave == 0) {
      const int nk = n < k ? n : k;
      const uint64_t key = lane < nk ? sh.S[lane] : 0ull;  // lane i: the i-th largest kept key
      const double s0 = (double)topk_key_score(sh.S[0]);
      const double w = key != 0 ? exp((double)topk_key_score(key) - s0) : 0.0;
      double incl = w;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const double total = __shfl(incl, 63);
      if (key != 0 && incl - w < (double)p.top_p * total) {
        bi = topk_key_id(key);
        bv = topk_key_score(key) + noise_of(bi);
      }
    }
  } else {
    for (int i = tid; i < n; i += kTopkMergeThreads) {
      const uint64_t key = sh.F[i];
      if (key == 0 || key < tau) continue;
      const int32_t id = topk_key_id(key);
      merge_best(bv, bi, topk_key_score(key) + noise_of(id), id);
    }
  }
  wave_best(bv, bi);
  if (lane == 0) {
    sh.red_v[wave] = bv;
    sh.red_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 0; w < kTopkMergeThreads / 64; ++w) merge_best(bv, bi, sh.red_v[w], sh.red_i[w]);
    p.out_idx[b] = bi;
  }
}

hipError_t launch_topk_merge(const StreamParams& p, hipStream_t stream) {
  if (p.n_tiles > kTopkMergeThreads || p.top_k < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(p.B), dim3(kTopkMergeThreads), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Conventional comparator, not the method: the softmax pipeline the fused
// sampler replaces [readus.org FlashSampling summary, the essay part: the
// softmax pipeline exponentiates every score, normalizes, and scans the
// cumulative array to pick a token].  Over stored logits, three launches:
//   1. stats (segment, row): segment max and sum of exp(s - max), allowed ids;
//   2. probs (segment, row): the row's max and total from the segment stats;
//      p = exp(s - m) / Z written over the logits (0 for masked ids), and the
//      segment's sum of the written p;
//   3. search (row): one uniform u per row and step, from word 0 of Philox at
//      counter (0x80000000, row, step); the segment where the running sum of
//      segment sums passes u * total; inside it, block-wide scans find the
//      first id whose running sum passes the remainder.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void cdf_segment(const CdfParams& p, int seg, int64_t& q_lo, int64_t& q_hi) {
  const int64_t nq = (p.V + 3) / 4;
  q_lo = (int64_t)seg * nq / p.n_seg;
  q_hi = (int64_t)(seg + 1) * nq / p.n_seg;
}

// Allowed-id bits of quad q (ids 4q .. 4q+3) of row b.
__device__ __forceinline__ uint32_t cdf_bits(const CdfParams& p, int b, int64_t q) {
  const int v0 = (int)(q * 4);
  uint32_t bits = p.mask ? (p.mask[(int64_t)b * p.ldm + (v0 >> 5)] >> (uint32_t)(v0 & 31)) & 0xFu : 0xFu;
  const int left = p.V - v0;
  if (left < 4) bits &= (1u << left) - 1u;
  return bits;
}

// Block-wide merge of (m, z) states; the result is valid in every thread.
__device__ __forceinline__ void cdf_block_lse(float& m, float& z, float* sm, float* sz) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off), oz = __shfl_xor(z, off);
    lse_merge(m, z, om, oz);
  }
  __syncthreads();
  if (lane == 0) {
    sm[wave] = m;
    sz[wave] = z;
  }
  __syncthreads();
  m = -INFINITY;
  z = 0.0f;
  for (int w = 0; w < kWaves; ++w) lse_merge(m, z, sm[w], sz[w]);
}

__global__ void __launch_bounds__(kThreads) cdf_stats_kernel(const CdfParams p) {
  __shared__ float sm[kWaves], sz[kWaves];
  const int seg = blockIdx.x, b = blockIdx.y;
  const float* row = p.logits + (int64_t)b * p.ldl;
  int64_t q_lo, q_hi;
  cdf_segment(p, seg, q_lo, q_hi);
  float m = -INFINITY, z = 0.0f;
  for (int64_t q = q_lo + threadIdx.x; q < q_hi; q += kThreads) {
    const f32x4_t x = *(const f32x4_t*)(row + q * 4);  // rows are padded to whole quads
    const uint32_t bits = cdf_bits(p, b, q);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((bits >> i) & 1u) lse_push(m, z, x[i] * p.inv_t);
  }
  cdf_block_lse(m, z, sm, sz);
  if (threadIdx.x == 0) {
    p.seg_m[(int64_t)b * kCdfMaxSeg + seg] = m;
    p.seg_z[(int64_t)b * kCdfMaxSeg + seg] = z;
  }
}

__global__ void __launch_bounds__(kThreads) cdf_probs_kernel(const CdfParams p) {
  __shared__ float sm[kWaves], sz[kWaves];
  const int seg = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = -INFINITY, z = 0.0f;
  for (int i = threadIdx.x; i < p.n_seg; i += kThreads)
    lse_merge(m, z, p.seg_m[(int64_t)b * kCdfMaxSeg + i], p.seg_z[(int64_t)b * kCdfMaxSeg + i]);
  cdf_block_lse(m, z, sm, sz);
  const float inv_z = z > 0.0f ? 1.0f / z : 0.0f;
  float* row = p.logits + (int64_t)b * p.ldl;
  int64_t q_lo, q_hi;
  cdf_segment(p, seg, q_lo, q_hi);
  float acc = 0.0f;
  for (int64_t q = q_lo + threadIdx.x; q < q_hi; q += kThreads) {
    f32x4_t x = *(const f32x4_t*)(row + q * 4);
    const uint32_t bits = cdf_bits(p, b, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ((bits >> i) & 1u) ? __expf(x[i] * p.inv_t - m) * inv_z : 0.0f;
      acc += x[i];
    }
    *(f32x4_t*)(row + q * 4) = x;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  __syncthreads();
  if (lane == 0) sm[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < kWaves; ++w) t += sm[w];
    p.seg_p[(int64_t)b * kCdfMaxSeg + seg] = t;
  }
}

__global__ void __launch_bounds__(kThreads) cdf_search_kernel(const CdfParams p) {
  __shared__ float s_wave[kWaves];
  __shared__ int s_seg, s_pick, s_last;
  __shared__ float s_rem;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* row = p.logits + (int64_t)b * p.ldl;
  if (threadIdx.x == 0) {
    s_pick = INT32_MAX;
    s_last = -1;
  }
  if (wave == 0) {  // running sum over segments (n_seg <= 64: one lane each)
    const float ps = lane < p.n_seg ? p.seg_p[(int64_t)b * kCdfMaxSeg + lane] : 0.0f;
    float incl = ps;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const float total = __shfl(incl, 63);
    const Philox4 r = philox4x32_10(p.seed_lo, p.seed_hi, 0x80000000u, (uint32_t)b, p.step_lo, p.step_hi);
    const float u = (float)(((double)r.w[0] + 1.0) / 4294967297.0);
    const float target = u * total;
    // the first segment with mass whose running sum passes the target; if
    // rounding leaves the running sum at the total, the last one with mass;
    // none (-1) if the row has no allowed id
    const uint64_t pass = __ballot(incl > target && ps > 0.0f);
    const uint64_t pos = __ballot(ps > 0.0f);
    const int j = pos == 0 ? -1 : (pass != 0 ? __builtin_ctzll(pass) : 63 - __builtin_clzll(pos));
    const float excl = j > 0 ? __shfl(incl, j - 1) : 0.0f;
    if (lane == 0) {
      s_seg = j;
      s_rem = target - excl;
    }
  }
  __syncthreads();
  const int j = s_seg;
  if (j < 0) {
    if (threadIdx.x == 0) p.out_idx[b] = -1;
    return;
  }
  const float rem = s_rem;
  int64_t q_lo, q_hi;
  cdf_segment(p, j, q_lo, q_hi);
  const int v_lo = (int)(q_lo * 4);
  const int v_hi = (int)(q_hi * 4 < p.V ? q_hi * 4 : p.V);
  float base = 0.0f;  // running sum before the current block of kThreads ids
  for (int v0 = v_lo; v0 < v_hi; v0 += kThreads) {
    const int v = v0 + threadIdx.x;
    const float x = v < v_hi ? row[v] : 0.0f;
    float incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    float before = base;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (x > 0.0f) {
      if (before + incl > rem) atomicMin(&s_pick, v);
      atomicMax(&s_last, v);
    }
    for (int w = 0; w < kWaves; ++w) base += s_wave[w];
    __syncthreads();
    if (s_pick != INT32_MAX) break;  // uniform: read after the barrier
  }
  if (threadIdx.x == 0) p.out_idx[b] = s_pick != INT32_MAX ? s_pick : s_last;
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
// LDS plan of a streaming launch: H resident when it fits (after the mask),
// else k-chunks (double-buffered when two fit); the tile's mask words are
// staged when they fit beside H.  Prefers the layouts the fast driver takes.
bool plan_stream(StreamParams& p, StreamConfig& cfg, int epi) {
  if (!cfg.dot && cfg.nb > 4) {
    // the wide kernel: its own H layout; the plain sampling epilogue, no mask,
    // one sample per row, d a multiple of its k-chunk ring
    if (epi != EPI_FLAT || p.mask || p.samples > 1 || p.d % wide_kmult(cfg.nb) != 0 || p.B > 16 * cfg.nb) return false;
    p.h_rows = p.B;
    p.h_rowstride = wide_pieces(cfg.nb) * 16;
    p.nsub = p.d / 256;
    p.cs = 1;
    p.nchunk = p.d / (32 * wide_ksteps(cfg.nb));
    p.nbuf = kWideHBufs;
    p.mask_words = 0;
    p.mask_lds_off = 0;
    p.noise_pitch = 0;
    p.noise_lds_off = 0;
    cfg.fast = true;
    cfg.rm = 0;
    p.tile_ratio = 0;
    cfg.lds_bytes = kWideHBufs * wide_bufbytes(cfg.nb);  // also covers the final reduction's scratch
    return cfg.lds_bytes <= kLdsMax;
  }
  if (epi == EPI_TOPK && (cfg.dot || p.n_tiles > kTopkMergeThreads)) return false;  // MFMA kernels only
  const int Bp = cfg.dot ? cfg.bd : cfg.nb * 16;
  const int hr = cfg.dot ? cfg.bd : (p.B < Bp ? p.B + 1 : Bp);
  p.h_rows = hr;
  p.nsub = (p.d + 255) / 256;
  const int scratch = epi == EPI_TOPK ? topk_finish_lds(cfg.nb) : kWaves * Bp * 16;
  auto rowstride = [](int cs) { return cs * 512 + 16; };
  const int64_t tile_rows = 16 * ((p.n_mblocks + p.n_tiles - 1) / p.n_tiles);  // largest tile
  // mask words of the largest tile (tile rows are a whole number of 16-row blocks)
  int mask_bytes = 0;
  p.mask_words = 0;
  if (p.mask) {
    const int64_t words = tile_mask_words(p.n_mblocks, p.n_tiles);
    const int64_t bytes = ((int64_t)p.B * words * 4 + 15) / 16 * 16;
    if (bytes > kMaskLdsMax) return false;
    p.mask_words = (int)words;
    mask_bytes = (int)bytes;
  }
  const int budget = kLdsMax - mask_bytes;
  // Whole H resident where it fits, for the sampling epilogues only up to 16
  // rows at d <= 2048 (small decode B=32 on MI355X: 109.7 us resident, 106.7
  // chunk-outer) and at d > 2048 only without a mask and if the tile's noise
  // table fits beside it (without it the resident kernel runs Philox in its
  // epilogue: mid decode B=15 and 16, 205.7 us, against 202.1 chunk-outer; with
  // a mask, d=5120, B=1 and 8: 265.1 and 268.7 us, against 260.5 and 261.0).
  // The stored-logits epilogue and the dot-product kernel use no table.
  const bool table_fits = (int64_t)hr * rowstride(p.nsub) + (int64_t)p.B * (tile_rows + 4) * 4 <= budget;
  // The top-k epilogue runs no Philox in its loop and needs no table: resident
  // H up to 16 rows without a mask.
  const bool prefer_resident =
      epi == EPI_STORE || cfg.dot ||
      (p.nsub <= 8 ? p.B <= 16 : (epi == EPI_TOPK ? p.B <= 16 : table_fits) && p.mask == nullptr);
  if ((int64_t)hr * rowstride(p.nsub) <= budget && prefer_resident) {
    p.cs = p.nsub;
    p.nchunk = 1;
    p.nbuf = 1;
  } else {
    int cs = 0;
    auto fits2 = [&](int c) {
      return (int64_t)2 * hr * rowstride(c) <= budget && hr * c * 32 <= kMaxStagePieces * kThreads;
    };
    if (p.nsub % kFastRingChunked == 0 && fits2(kFastRingChunked)) {
      cs = kFastRingChunked;
    } else {
      for (int c = p.nsub; c >= 1; --c)
        if (fits2(c)) {
          cs = c;
          break;
        }
    }
    if (cs > 0) {
      p.cs = cs;
      p.nbuf = 2;
    } else if ((int64_t)hr * rowstride(1) <= budget && hr * 32 <= kMaxStagePieces * kThreads) {
      p.cs = 1;
      p.nbuf = 1;
    } else {
      return false;
    }
    p.nchunk = (p.nsub + p.cs - 1) / p.cs;
    if (p.nchunk == 1) p.nbuf = 1;
  }
  p.h_rowstride = rowstride(p.cs);
  const int hbytes = p.nbuf * hr * p.h_rowstride;
  p.mask_lds_off = hbytes;
  int total = hbytes + mask_bytes;
  // Noise table: the tile's Gumbel noise for the B rows, computed before the
  // stream starts (every lane does useful work there, while in the epilogue a
  // 16-row MFMA block with B < 16 would compute noise for padding rows).
  p.noise_pitch = 0;
  p.noise_lds_off = 0;
  const bool full_k = p.d % 256 == 0;
  if (p.nchunk == 1)
    cfg.fast = full_k && p.nsub % kFastRingResident == 0;
  else
    cfg.fast = full_k && p.cs == kFastRingChunked && p.nbuf == 2 && p.nsub % kFastRingChunked == 0;
  // Chunked H with the fast driver: the chunk-outer kernel, whose passes cover
  // up to kouter_max_rounds rounds.
  cfg.rm = 0;
  if (!cfg.dot && cfg.fast && p.nchunk > 1) {
    // XCD-weighted tiles where the caller allows them (tile_ratio set on entry):
    // plain sampling without a mask or its stored-logits pass (the same tiles
    // keep the stored logits equal bit for bit to the fused path's), whole XCD
    // sets of tiles, at least 16 blocks a tile (with fewer, one more block can
    // add a round to a tile)
    if (p.tile_ratio != 0 && !((epi == EPI_FLAT || epi == EPI_STORE || epi == EPI_TOPK) && p.mask == nullptr &&
                               p.group_tiles == 0 &&
                               p.n_tiles % 8 == 0 && p.n_mblocks >= 16 * (int64_t)p.n_tiles))
      p.tile_ratio = 0;
    int64_t max_blocks = 0;
    for (int t = 0; t < p.n_tiles; ++t) {
      const int64_t n = tile_lo(t + 1, p.n_mblocks, p.n_tiles, p.tile_ratio) - tile_lo(t, p.n_mblocks, p.n_tiles, p.tile_ratio);
      if (n > max_blocks) max_blocks = n;
    }
    const int64_t rounds = (max_blocks + kWaves - 1) / kWaves;
    // passes of equal length: a short last pass would leave waves re-reading
    // their last block for the rounds they do not own
    const int cap = kouter_max_rounds(epi, cfg.nb, epi != EPI_STORE && p.mask != nullptr);
    const int64_t npass = (rounds + cap - 1) / cap;
    cfg.rm = (int)((rounds + npass - 1) / npass);
  }
  if (cfg.rm == 0) p.tile_ratio = 0;
  // The tile's noise table, for rows of more than 8 sub-blocks (d > 2048).  At
  // d <= 2048 the kernel running Philox in its epilogue, with its sub-blocks
  // rotated per workgroup, measured faster on MI355X (small decode B=1..16:
  // 118 -> 108 us); at d=4096 the table kernel is faster (195 vs 204 us).
  if (!cfg.dot && cfg.fast && cfg.rm == 0 && (epi == EPI_FLAT || epi == EPI_GROUP) && p.nsub > 8) {
    const int pitch = (int)tile_rows + 4;
    const int64_t nbytes = (int64_t)p.B * pitch * 4;
    if (total + nbytes <= kLdsMax) {
      p.noise_pitch = pitch;
      p.noise_lds_off = total;
      total += (int)nbytes;
    }
  }
  cfg.lds_bytes = total > scratch ? total : scratch;
  return true;
}

// The streaming pass, then (sampling epilogues) the reduction over its tiles.
hipError_t launch_stream(const StreamParams& p, const StreamConfig& cfg, int epi, hipStream_t stream,
                         hipEvent_t ev_before, hipEvent_t ev_after) {
  hipError_t e;
  const dim3 rgrid((p.B + kWaves - 1) / kWaves);
  if (ev_before && (e = hipEventRecord(ev_before, stream)) != hipSuccess) return e;
  switch (epi) {
    case EPI_FLAT:
      e = launch_stream_epi<EPI_FLAT>(p, cfg, stream);
      if (e != hipSuccess) return e;
      if (ev_after && (e = hipEventRecord(ev_after, stream)) != hipSuccess) return e;
      hipLaunchKernelGGL(reduce_tiles_kernel<EPI_FLAT>, rgrid, dim3(kThreads), 0, stream, p.B, p.n_tiles, p.ws_val,
                         p.ws_idx, nullptr, nullptr, p.out_idx, nullptr, p.n_tiles, (int64_t)0);
      return hipGetLastError();
    case EPI_GROUP:
      e = launch_stream_epi<EPI_GROUP>(p, cfg, stream);
      if (e != hipSuccess) return e;
      if (ev_after && (e = hipEventRecord(ev_after, stream)) != hipSuccess) return e;
      if (p.group_tiles > 0) {  // one summary per group: out_sum is [groups][out_stride]
        const dim3 ggrid((p.B + kWaves - 1) / kWaves, p.n_tiles / p.group_tiles);
        hipLaunchKernelGGL(reduce_tiles_kernel<EPI_GROUP>, ggrid, dim3(kThreads), 0, stream, p.B, p.n_tiles,
                           p.ws_val, p.ws_idx, p.ws_m, p.ws_s, nullptr, p.out_sum, p.group_tiles, p.group_out_stride);
      } else {
        hipLaunchKernelGGL(reduce_tiles_kernel<EPI_GROUP>, rgrid, dim3(kThreads), 0, stream, p.B, p.n_tiles,
                           p.ws_val, p.ws_idx, p.ws_m, p.ws_s, nullptr, p.out_sum, p.n_tiles, (int64_t)0);
      }
      return hipGetLastError();
    case EPI_STORE:
      e = launch_stream_epi<EPI_STORE>(p, cfg, stream);
      if (e != hipSuccess) return e;
      return ev_after ? hipEventRecord(ev_after, stream) : hipSuccess;
    case EPI_TOPK:
      e = launch_stream_epi<EPI_TOPK>(p, cfg, stream);
      if (e != hipSuccess) return e;
      if (ev_after && (e = hipEventRecord(ev_after, stream)) != hipSuccess) return e;
      return launch_topk_merge(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sample_logits(const SampleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(sample_logits_kernel, dim3(p.n_tiles), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_tiles_kernel<EPI_FLAT>, dim3((p.B + kWaves - 1) / kWaves), dim3(kThreads), 0, stream, p.B,
                     p.n_tiles, p.ws_val, p.ws_idx, nullptr, nullptr, p.out_idx, nullptr, p.n_tiles, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_topk_sample(const TopkParams& p, hipStream_t stream) {
  const dim3 grid(p.n_seg, p.B);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cdf_sample(const CdfParams& p, hipStream_t stream) {
  const dim3 grid(p.n_seg, p.B);
  hipLaunchKernelGGL(cdf_stats_kernel, grid, dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(cdf_probs_kernel, grid, dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(cdf_search_kernel, dim3(p.B), dim3(kThreads), 0, stream, p);
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
