// fs_kernels.h -- host-visible launch interface of the FlashSampling kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsk {

// EPI_TOPK: the fused top-k pass -- per lane, a short list of the best scores
// it saw; per (row, tile) a merged list and a bound on what it dropped
// (see fs_stream.h), finished by topk_merge_kernel.
enum Epilogue { EPI_FLAT = 0, EPI_GROUP = 1, EPI_STORE = 2, EPI_TOPK = 3 };

struct GroupSummary {  // same layout as fs_group_summary_t
  float lse;
  float pmax;
  int32_t arg;
};

// Geometry and pointers of one streaming launch (one workgroup per vocab tile).
struct StreamParams {
  const uint16_t* H;
  int64_t ldh;
  const uint16_t* W;
  int64_t ldw;
  int B;
  int d;
  int64_t V;             // rows of W in this launch
  int64_t vocab_offset;  // global vocab id of W row 0 (noise and mask use global ids)
  int row_offset;        // global batch row of H row 0 (noise counter and mask row)
  // Several samples per row: batch row b of the launch is virtual row
  // r = vrow0 + b = h * samples + s of the call, drawing sample s of H row h
  // with noise at step + s (H then points at the call's first row).  With
  // samples == 1, batch row b is H row b.
  int samples;
  int vrow0;
  // Several vocabulary groups in one launch: group_tiles > 0 tiles per group,
  // each group group_blocks 16-row blocks long; tiles never straddle groups.
  int group_tiles;
  int64_t group_blocks;
  int64_t group_out_stride;  // summaries between consecutive groups in out_sum
  float inv_t;
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
  const uint32_t* mask;  // [B, ldm] words or null
  int64_t ldm;
  int n_tiles;        // = gridDim.x
  int64_t n_mblocks;  // ceil(V / 16)
  int nsub;           // ceil(d / 256): k sub-blocks of 256
  int cs;             // sub-blocks per LDS chunk of H
  int nchunk;         // ceil(nsub / cs)
  int nbuf;           // LDS buffers for H chunks (1 or 2)
  int h_rowstride;    // bytes per H row in LDS
  int h_rows;         // H rows per LDS buffer: the B rows of H, plus one zero row read by the
                      // padding lanes of a 16-wide MFMA block when B is not a multiple of 16
  int noise_pitch;    // > 0: the tile's Gumbel noise is precomputed into LDS, this many floats per row
  int noise_lds_off;  // byte offset of the noise table in LDS
  int mask_words;     // mask words per row staged in LDS (set whenever mask is non-null)
  int mask_lds_off;   // byte offset of the staged mask in LDS
  // per-tile results, [B][n_tiles]
  float* ws_val;
  int32_t* ws_idx;
  float* ws_m;
  float* ws_s;
  int32_t* out_idx;
  GroupSummary* out_sum;
  float* dbg_max;  // [B][n_tiles] or null
  int32_t* dbg_arg;
  float* logits;  // EPI_STORE: [B][ldl] fp32
  int64_t ldl;
  int tile_ratio;  // 0: equal tiles; else XCD-weighted tiles (see tile_lo)
  // EPI_TOPK: k, and the per-(row, tile) candidate lists, laid out as
  // topk_cand[(b * kTopkSlot + j) * n_tiles + tile]
  int top_k;
  uint64_t* topk_cand;
  float top_p;  // EPI_TOPK: nucleus of the kept ids (1: all of them)
  // Online grouped summaries (EPI_GROUP with group_tiles > 0): when ready is
  // not null, the tiles of launch group g start once ready[g] == ready_epoch,
  // waiting at most wait_ticks of the 100 MHz real-time clock; a tile that
  // gives up sets *status to 1 and does no work.
  const uint32_t* ready;
  uint32_t ready_epoch;
  uint64_t wait_ticks;
  int32_t* status;
};

struct SampleParams {  // unfused second pass: sample from stored logits
  const float* logits;
  int64_t ldl;
  int B;
  int64_t V;
  float inv_t;
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
  const uint32_t* mask;
  int64_t ldm;
  int n_tiles;
  float* ws_val;
  int32_t* ws_idx;
  int32_t* out_idx;
};

// Top-k sampling from stored fp32 logits (segment-parallel radix select, then a
// per-row finish).
struct TopkParams {
  const float* logits;  // [B][ldl], row b holds global batch row row_offset + b
  int64_t ldl;
  int B;
  int V;
  float inv_t;
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
  const uint32_t* mask;  // [*, ldm] words indexed by the global batch row, or null
  int64_t ldm;
  int row_offset;
  int top_k;
  int32_t* out_idx;  // [B]
  // selection workspace, zero between calls where noted
  int n_seg;           // segments per row (<= kTopkMaxSeg)
  uint32_t* hist;      // [B][kTopkBins] row histograms of key bits 31..20 (zero)
  uint64_t* cand;      // [B][kTopkCap] boundary-bin candidates (key << 32 | ~id)
  int32_t* cand_n;     // [B] candidate counts (zero)
  float* seg_val;      // [B][kTopkMaxSeg] segment maximizers
  int32_t* seg_idx;
  int32_t* bound;          // [B][4] row boundary: bin, count above, count inside, total
  uint32_t* arrive_hist;   // [B] arrival counters of the two launches (zero)
  uint32_t* arrive_coll;
};

// Conventional comparator (softmax, prefix sum, inverse-CDF search) over
// stored fp32 logits, overwritten in place by the probabilities.
struct CdfParams {
  float* logits;  // [B][ldl]: logits in, probabilities out
  int64_t ldl;
  int B;
  int V;
  float inv_t;
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
  const uint32_t* mask;  // [B, ldm] words or null
  int64_t ldm;
  int n_seg;       // segments per row (<= kCdfMaxSeg)
  float* seg_m;    // [B][kCdfMaxSeg] segment max of s
  float* seg_z;    // [B][kCdfMaxSeg] segment sum of exp(s - segment max)
  float* seg_p;    // [B][kCdfMaxSeg] segment sum of the written probabilities
  int32_t* out_idx;
};

// Kernel selection for a streaming launch.
struct StreamConfig {
  bool dot;     // dot-product kernel (else MFMA)
  int nb;       // MFMA: 16-wide batch blocks (1, 2, 4; 8 or 16: the wide kernel)
  int bd;       // dot: padded batch (1, 2)
  bool fast;    // straight-line fast driver (see fs_stream.h)
  int rm;       // chunked H with the fast driver: rounds per chunk-outer pass (0: round-major kernel)
  int lds_bytes;
};

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kLdsMax = 160 * 1024 - 256;  // leaves room for the kernels' static LDS
constexpr int kMaxStagePieces = 8;  // 16-byte H pieces per thread held for the next LDS chunk
constexpr int kDotMaxB = 2;
constexpr int kFastRingResident = 2;  // register ring depth of the fast driver, H resident (measured best)
constexpr int kFastRingChunked = 2;   // ... and with k-chunked H (chunks of exactly this many sub-blocks)
constexpr int kMfmaMaxB = 64;
// The wide kernel (65 .. kWideMaxB batch rows of the plain sampler, no mask):
// kWideWaves waves, each holding wide_mw(NB) x NB accumulator blocks (NB = 8
// up to 128 rows, 16 above; at NB = 16 the 80 blocks take all 256 AGPRs and
// 64 VGPRs); passes of up to kWideWaves * wide_mw(NB) vocab
// blocks; H in k-chunks of 32 wide_ksteps(NB), kWideHBufs LDS buffers of
// wide_bufbytes(NB); W register items of one chunk, wide_ring(NB) of them,
// each item's loads issued wide_lead(NB) chunks ahead (d must be a multiple
// of wide_kmult(NB)).
constexpr int kWideMaxB = 256;
constexpr int kWideWaves = 4;
constexpr int kWideHBufs = 3;
constexpr int wide_nb(int B) { return B <= 128 ? 8 : 16; }
constexpr int wide_mw(int nb) { return 5; }
constexpr int wide_ksteps(int nb) { return 2; }
constexpr int wide_pieces(int nb) { return wide_ksteps(nb) * 4 + 1; }
constexpr int wide_bufbytes(int nb) { return nb * 16 * wide_pieces(nb) * 16; }
constexpr int wide_ring(int nb) { return 4; }
constexpr int wide_lead(int nb) { return 2; }
constexpr int wide_kmult(int nb) { return 32 * wide_ksteps(nb) * wide_ring(nb); }
// s_waitcnt immediate that waits until at most n vector-memory loads of the
// wave are outstanding (expcnt and lgkmcnt left alone)
constexpr unsigned vmcnt_wait(int n) { return (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14) | 0x70u | 0xF00u; }
// Which 16 bytes of a row's 512-byte sub-block lane group g (0..3) loads with
// its load instruction e (0..7), and so which 8-value k chunk it feeds to MFMA
// step e (H is read with the same map): lane_base(g) + e * lane_step bytes.
//   0: each group a 128-byte run             (128 g + 16 e)
//   1: the four groups side by side          (16 g + 64 e)
//   2: two pairs side by side, one per half  (256 (g >> 1) + 16 (g & 1) + 32 e)
// One load instruction of a wave touches 64, 16 or 32 cache lines.  The map
// per kernel family is the measured best on gfx950.
constexpr int kLayoutTable = 0;     // round-major kernel with the tile's noise table in LDS
constexpr int kLayoutEpilogue = 1;  // round-major kernel, noise in the epilogue
constexpr int kLayoutStore = 0;     // round-major kernel storing the logits
constexpr int kLayoutKouter = 1;    // chunk-outer kernel
constexpr int kLayoutTopk = 0;      // round-major kernel with the top-k epilogue
constexpr int kLayoutKouterTopk = 1;  // chunk-outer kernel with the top-k epilogue
constexpr int kLayoutDot = 0;       // dot-product kernel
// Rounds per pass of the chunk-outer kernel (accumulator sets a wave keeps in
// registers), by epilogue, batch blocks and masking: the most that fit 256
// VGPRs without spilling, except the plain sampler at four batch blocks, where
// five rounds (one pass over the decode heads' tiles, 8 VGPRs spilled outside
// the chunk loop) measured faster than three.
constexpr int kouter_max_rounds(int epi, int nb, bool masked) {
  return (nb <= 2 || epi == EPI_STORE || ((epi == EPI_FLAT || epi == EPI_TOPK) && !masked)) ? 5 : 3;
}
// Fused top-k: each lane keeps its kTopkLane best (score, id) pairs; each
// workgroup merges its lanes' lists per batch row into kTopkLane entries plus
// one bound (kTopkSlot = kTopkLane + 1 words of the candidate buffer).  k up to
// kTopkFusedMax runs fused; larger k stores the logits and selects from them.
constexpr int kTopkLane = 4;
constexpr int kTopkSlot = kTopkLane + 1;
// LDS bytes the end of a top-k streaming kernel uses (the H buffers, free by
// then): every wave's list and bound for each of the 16 NB batch columns, which
// the workgroup merges into one list per tile.
constexpr int topk_finish_lds(int nb) { return kWaves * nb * 16 * kTopkSlot * 8; }
constexpr int kTopkFusedMax = 64;
constexpr int kTopkMergeThreads = 256;
constexpr int kTopkMergeCap = 4096;      // candidate keys a row's merge holds in LDS
constexpr int kTopkMergeMaxTiles = 1024;
constexpr int kMaskLdsMax = 16 * 1024;  // LDS bytes for the staged tile mask

// First 16-row block of tile t of n_tiles over n_mblocks blocks.  ratio == 0:
// equal tiles.  ratio > 0: a tile of even index takes ratio / 1000 times the
// blocks of an odd one.  Workgroup t runs on XCD t mod 8, and on MI355X the odd
// XCDs streamed 2.6% slower than the even ones (mid decode B=64, two boxes):
// their workgroups finished last.  Used for the chunk-outer kernel only (it
// gained 1.0-1.3 us at mid decode B=24..64; the resident kernel and the group
// summaries gained nothing).
constexpr int kXcdTileRatio = 1026;
__host__ __device__ inline int64_t tile_lo(int64_t t, int64_t n_mblocks, int n_tiles, int ratio) {
  if (ratio == 0) return t * n_mblocks / n_tiles;
  const auto w = [ratio](int64_t u) { return 1000 * (u / 2) + (int64_t)ratio * ((u + 1) / 2); };
  return n_mblocks * w(t) / w(n_tiles);
}
constexpr int kTopkBins = 4096;    // first-level bins of the top-k radix select (key bits 31..20)
constexpr int kTopkCap = 2048;     // boundary-bin ids the segment-parallel selection gathers per row
constexpr int kTopkMaxSeg = 64;    // segments per row in the top-k launches
constexpr int kCdfMaxSeg = 64;     // segments per row in the comparator's launches

// Mask words per row staged for the largest tile of a launch.
inline int64_t tile_mask_words(int64_t n_mblocks, int n_tiles) {
  return 16 * ((n_mblocks + n_tiles - 1) / n_tiles) / 32 + 2;
}

// Fills the K/LDS geometry fields of p and the LDS size of cfg; returns false
// if the shape does not fit the kernels' LDS budget.
bool plan_stream(StreamParams& p, StreamConfig& cfg, int epi);

// ev_before / ev_after (may be null): recorded on `stream` right before and
// right after the streaming kernel (before the tile reduction), for timing.
hipError_t launch_stream(const StreamParams& p, const StreamConfig& cfg, int epi, hipStream_t stream,
                         hipEvent_t ev_before = nullptr, hipEvent_t ev_after = nullptr);
template <int EPI>
hipError_t launch_stream_epi(const StreamParams& p, const StreamConfig& cfg, hipStream_t stream);
hipError_t launch_sample_logits(const SampleParams& p, hipStream_t stream);
hipError_t launch_topk_merge(const StreamParams& p, hipStream_t stream);
hipError_t launch_topk_sample(const TopkParams& p, hipStream_t stream);
hipError_t launch_cdf_sample(const CdfParams& p, hipStream_t stream);
hipError_t launch_group_combine(const GroupSummary* s, int n_groups, int B, uint64_t seed, uint64_t step, int mode,
                                int32_t* out_idx, hipStream_t stream);
hipError_t launch_debug_philox(uint64_t seed, uint64_t step, uint32_t row, int64_t v0, int64_t n, uint32_t* r_out,
                               float* g_out, hipStream_t stream);
hipError_t launch_debug_gumbel_bits(uint64_t r0, int64_t n, float* g_out, hipStream_t stream);
hipError_t launch_debug_gumbel_scan(unsigned long long* stats, hipStream_t stream);

}  // namespace fsk
