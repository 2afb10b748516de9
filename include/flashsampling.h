/*
 * flashsampling.h -- C ABI of the MI355X (gfx950) FlashSampling library.
 *
 * FlashSampling draws one token per row from softmax(H W^T / T) without ever
 * writing the [B, V] logits to HBM: the LM-head product is computed tile by
 * tile on chip, Gumbel noise is added to every logit, each workgroup keeps one
 * (value, index) maximizer per row for its vocabulary tile, and a small
 * reduction over tiles gives the sample.  This is exact because argmax
 * decomposes over any partition of the vocabulary, and adding i.i.d. standard
 * Gumbel noise before an argmax draws exactly from the softmax.
 *   [FlashSampling: Fast and Memory-Efficient Exact Sampling, arXiv 2603.15854,
 *    abstract; readus.org FlashSampling summary, sections "Gumbel Max Trick"
 *    and on the two-stage FMMS kernel]
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; they must
 *     stay valid until the work enqueued on `stream` has completed.  The
 *     library never frees or retains them.
 *   - bf16 tensors are passed as uint16_t bit patterns (the upper half of an
 *     IEEE binary32).  Matrices are row-major with an explicit row stride in
 *     elements (ld*), which must be a multiple of 8; H and W must be 16-byte
 *     aligned (the kernels use 128-bit loads).
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Calls validate their arguments synchronously, enqueue work and return
 *     without waiting.  Faults inside kernels surface at the caller's next
 *     synchronisation, as with any HIP launch.
 *   - Return value: FS_OK or a negative FS_ERR_* code; fs_last_error() then
 *     holds a message (thread-local).  On an error nothing is enqueued.
 *   - A context owns its device workspace (tile winners, counters).  Calls on
 *     one context must not overlap in time: use one context per stream.
 *   - Noise is a pure function of (seed, step, row, vocab id), so results do
 *     not depend on tiling, code path or how rows are split across calls
 *     (up to fp32 summation order in the logits).
 */
#ifndef FLASHSAMPLING_H_
#define FLASHSAMPLING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FS_OK = 0,
  FS_ERR_INVALID_ARG = -1, /* a pointer, size, stride or value is out of its documented range */
  FS_ERR_UNSUPPORTED = -2, /* a combination the library does not implement */
  FS_ERR_CAPACITY = -3,    /* a size exceeds what the context was created for */
  FS_ERR_HIP = -4          /* the HIP runtime reported an error (message in fs_last_error) */
};

enum { FS_COMBINE_GUMBEL = 0, FS_COMBINE_MAX = 1 };

/* Code path selection for the streaming kernels (testing and measurement). */
enum { FS_PATH_AUTO = 0, FS_PATH_DOT = 1, FS_PATH_MFMA = 2 };

typedef struct fs_ctx fs_ctx;

/* Per-row summary of one vocabulary group (grouped / online variant).
 *   lse  = log sum_{allowed v in group} exp(logit_v / T)    (-inf if none allowed)
 *   pmax = max_{allowed v in group} (logit_v / T + g_v)      (-inf if none allowed)
 *   arg  = global vocab id attaining pmax, lowest on ties     (-1 if none allowed)
 * The group's log-sum-exp is its "captain"; a Gumbel draw over captains picks
 * the group, which is exact by hierarchical factorization of the categorical.
 *   [arXiv 2603.15854 abstract; readus.org summary, section "Group Gumbel Max"] */
typedef struct {
  float lse;
  float pmax;
  int32_t arg;
} fs_group_summary_t;

/* Create a context on `device` for calls with B <= max_B, V <= max_V and
 * top_k <= max_top_k.  Allocates the device workspace once; no later call
 * allocates device memory.  With max_top_k > 0 the workspace holds the fused
 * top-k's candidate lists (min(max_B, 64) rows x 256 tiles x 40 bytes);
 * with max_top_k > 64 also min(max_B, 64) rows of max_V fp32 scores.
 * *out is set to NULL on failure. */
int fs_create(fs_ctx** out, int device, int max_B, int64_t max_V, int max_top_k);

/* Release a context and its workspace (NULL is ignored).  Work that used the
 * context must have completed. */
void fs_destroy(fs_ctx* ctx);

/* Message for the last non-OK status returned on the calling thread. */
const char* fs_last_error(void);

/* Number of vocabulary tiles (= workgroups) and the tile bounds used by
 * fs_fmms_sample for these sizes when it reports tile maxima.  bounds, if not
 * NULL, receives n_tiles + 1 ascending vocab ids: tile i covers
 * [bounds[i], bounds[i+1]).  Tiles are contiguous and balanced in units of 16
 * vocab rows.  Calls that do not report tile maxima may size the tiles per
 * XCD instead (the tiling changes only the order of the fp32 sums behind the
 * logits, so the sampled ids agree except at near ties). */
int fs_fmms_tiling(fs_ctx* ctx, int B, int d, int64_t V, int path, int64_t* n_tiles, int64_t* bounds);

/* Fused LM-head matmul + sample (FMMS).
 *   H [B, d] bf16, row stride ldh;  W [V, d] bf16, row stride ldw.
 *   logit[b][v] = sum_k H[b][k] W[v][k]   (bf16 products, fp32 accumulation)
 *   s = logit * (1/T); masked ids -> -inf; with top_k > 0 only the top_k
 *   largest s of the row's allowed ids are kept (ties at the boundary by lower
 *   id); p = s + g(seed, step, b, v); out_idx[b] = argmax_v p (lowest id on
 *   ties; -1 if the row has no allowed id).
 *   g is standard Gumbel noise: r = word (v & 3) of Philox4x32-10 with key
 *   (lo32 seed, hi32 seed) and counter (v >> 2, b, lo32 step, hi32 step);
 *   u = (r + 1) / (2^32 + 1); g = -log(-log u).
 *   [readus.org summary, code guide: API (weights, hidden states, temperature,
 *    seed), RNG (Philox keyed by seed and coordinates), floating point (the u
 *    formula); section on Top-K and masking]
 * mask: NULL, or [B, ldm] uint32 words with ldm >= ceil(V/32): bit (v & 31)
 *       of word (v >> 5) of row b set means id v is allowed.
 * temperature: finite and > 0.
 * out_idx: [B] int32 device.
 * tile_max, tile_arg: NULL, or [B, n_tiles] (n_tiles from fs_fmms_tiling)
 *       receiving each tile's maximum perturbed score and its id (top_k == 0
 *       only); for tests.
 * path: FS_PATH_AUTO, or force the dot-product or MFMA streaming kernel.
 * top_k: 0 (off), or 1 <= top_k <= max_top_k.  With top_k <= 64 (and not the
 *       dot-product path) the top-k is fused: the streaming pass keeps, per
 *       batch row and vocabulary tile, the 4 best scores it saw and a bound
 *       on the scores it dropped; a second launch per batch chunk
 *       selects the row's top k from those lists, rescoring a tile from H and
 *       W when its bound reaches the k-th score, and draws the Gumbel-max
 *       among them.  No [B, V] scores reach HBM.  Larger k stores each
 *       chunk's fp32 scores in the context's workspace (max_top_k > 64 at
 *       fs_create) and selects from them.
 * Requires 1 <= B <= max_B, 8 <= d, d % 8 == 0, 1 <= V <= max_V < 2^31. */
int fs_fmms_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                   int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                   const uint32_t* mask, int64_t ldm, int top_k, int32_t* out_idx, float* tile_max,
                   int32_t* tile_arg, int path);

/* Top-k, then top-p (nucleus) sampling, fused.
 *   The top_k largest scores s of the row's allowed ids are kept as in
 *   fs_fmms_sample; sorted by s (descending, lower id first), a kept id stays
 *   in the nucleus while the weight exp(s - s_max) of the ids ahead of it,
 *   summed in fp64, is below top_p times the weight of all kept ids -- the
 *   shortest prefix holding top_p of their mass.  out_idx[b] is the Gumbel-max
 *   over the nucleus with the same per-id noise (-1 if no id is allowed).
 *   top_p = 1 gives fs_fmms_sample's top-k sample.
 *   [nucleus sampling as defined by Holtzman et al., "The Curious Case of
 *    Neural Text Degeneration", ICLR 2020; cjcn.com.cn and news.neo-ai.one
 *    FlashSampling articles: the method is compatible with top-p sampling]
 * Requires 1 <= top_k <= min(max_top_k, 64) (FS_ERR_UNSUPPORTED above 64),
 * 0 < top_p <= 1, path FS_PATH_AUTO or FS_PATH_MFMA; other arguments as in
 * fs_fmms_sample. */
int fs_fmms_sample_top_p(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                         int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                         const uint32_t* mask, int64_t ldm, int top_k, float top_p, int32_t* out_idx, int path);

/* Several samples per row from one pass over W.
 *   out_idx [B, num_samples] int32 (row-major): out_idx[b * num_samples + s] is
 *   the id fs_fmms_sample returns for row b at step `step + s` (64-bit
 *   wrap-around), i.e. num_samples independent draws from the same
 *   softmax(logits / T) with the noise streams of consecutive steps.  W is
 *   read once per 64 (row, sample) pairs.  Other arguments as in
 *   fs_fmms_sample; no top-k or tile maxima here.
 *   [readus.org summary, code guide item 1: the API takes a number of samples]
 * Requires num_samples >= 1 and B * num_samples < 2^31. */
int fs_fmms_sample_multi(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                         int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                         const uint32_t* mask, int64_t ldm, int num_samples, int32_t* out_idx, int path);

/* Unfused comparison path: the same LM-head product written to HBM as fp32
 * logits, then a separate sampling kernel reads them back and applies the
 * same scaling, mask, top-k, noise and argmax.  Same arguments and result as
 * fs_fmms_sample (identical ids when the same path computes the logits).
 * logits_ws: [B, ldl] fp32 device buffer with ldl >= V, ldl % 4 == 0,
 *       16-byte aligned; receives the unscaled logits. */
int fs_unfused_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                      int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                      const uint32_t* mask, int64_t ldm, int top_k, int32_t* out_idx, float* logits_ws,
                      int64_t ldl, int path);

/* Conventional comparator, not the method: the softmax pipeline the fused
 * sampler replaces.  The LM-head product goes to logits_ws as fp32 logits, a
 * softmax of s = logit / T over the allowed ids overwrites them in place with
 * probabilities (masked ids get 0), and an inverse-CDF search draws the sample:
 * with u = (r + 1) / (2^32 + 1), r = word 0 of Philox4x32-10(key = seed,
 * counter = (0x80000000, b, lo32 step, hi32 step)), out_idx[b] is the first id
 * whose running sum of probabilities exceeds u times their total (-1 if the
 * row has no allowed id).  A draw from the same softmax(logits / T) as
 * fs_fmms_sample, but not the same draw.
 *   [readus.org summary, the essay part on the softmax pipeline: exponentiate,
 *    normalize and scan a cumulative array]
 * logits_ws: [B, ldl] fp32 device buffer, ldl >= V, ldl % 4 == 0, 16-byte
 *       aligned; holds the probabilities on return.
 * Other arguments and requirements as in fs_fmms_sample (no top-k). */
int fs_softmax_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                      int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                      const uint32_t* mask, int64_t ldm, int32_t* out_idx, float* logits_ws, int64_t ldl, int path);

/* Grouped / online variant: summary of one vocabulary group.
 *   W_group [G, d] bf16 (row stride ldw) holds the LM-head rows of global vocab
 *   ids [vocab_offset, vocab_offset + G); noise uses the global ids, so the
 *   group's pmax/arg are exactly the flat sampler's restricted to the group.
 *   mask: NULL or the full-vocabulary mask [B, ldm] (word (v >> 5) of global
 *   id v); vocab_offset % 32 == 0.
 *   out: [B] device summaries.  [arXiv 2603.15854 abstract: grouped variants
 *   for online and tensor-parallel settings; readus.org summary, "Group Gumbel
 *   Max": stream groups, keep each group's captain, discard the rest] */
int fs_group_summary(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W_group,
                     int64_t ldw, int B, int d, int64_t vocab_offset, int64_t G, float temperature,
                     uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm, fs_group_summary_t* out,
                     int path);

/* Summaries of n_groups consecutive groups of G ids each in one launch:
 *   W [n_groups * G, d] bf16 (row stride ldw) holds the LM-head rows of global
 *   ids [vocab_offset, vocab_offset + n_groups * G); out [n_groups, B]
 *   (group-major) receives, for group k, what fs_group_summary returns for
 *   W + k * G * ldw at vocab_offset + k * G.  For callers that hold several
 *   groups at once (a vocabulary shard, or every group of a step): H is staged
 *   once per pass over many groups' rows instead of once per group.
 *   mask as in fs_group_summary (full-vocabulary words).
 *   [arXiv 2603.15854 abstract: grouped variants for online and
 *    tensor-parallel settings; readus.org summary, "Group Gumbel Max"]
 * Requires G % 16 == 0, n_groups >= 1, vocab_offset % 32 == 0 and
 * vocab_offset + n_groups * G < 2^31. */
int fs_group_summaries(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                       int B, int d, int64_t vocab_offset, int64_t G, int n_groups, float temperature, uint64_t seed,
                       uint64_t step, const uint32_t* mask, int64_t ldm, fs_group_summary_t* out, int path);

/* Online grouped producer: fs_group_summaries whose groups are consumed as
 * they are published.  The tiles of group k (the launch gives each group an
 * equal share of the GPU's workgroups) start streaming only once ready[k]
 * equals epoch, so a producer -- the host writing a flag in pinned host
 * memory, or work on another stream -- can hand over group k's rows of W while
 * the launch already runs on the groups before it; with every flag already set
 * it is fs_group_summaries.
 *   ready [n_groups] uint32, device memory or pinned host memory mapped into
 *     the device (read with system-scope acquire loads); the producer writes
 *     epoch to ready[k] after group k's rows of W are in place (a release).
 *   max_wait_us: bound of each tile's wait (at most 60 s).  A tile whose flag
 *     does not arrive in time does no work and sets *status (device int32,
 *     caller-owned, not cleared by this call) to 1; that group's summaries
 *     are then unspecified.
 *   Everything else as in fs_group_summaries.
 *   [arXiv 2603.15854 abstract: grouped variants for online settings;
 *    readus.org summary, "Group Gumbel Max"]
 * Errors as fs_group_summaries; also FS_ERR_INVALID_ARG for a NULL ready or
 * status. */
int fs_group_summaries_online(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W,
                              int64_t ldw, int B, int d, int64_t vocab_offset, int64_t G, int n_groups,
                              float temperature, uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm,
                              const uint32_t* ready, uint32_t epoch, uint32_t max_wait_us, int32_t* status,
                              fs_group_summary_t* out, int path);

/* Combine per-group summaries s [n_groups, B] (group-major) into one sample
 * per row.
 *   FS_COMBINE_GUMBEL: k* = argmax_k (lse_k + g'_k) with g'_k the Gumbel
 *     transform of word 0 of Philox4x32-10(key = seed, counter = (0x40000000 | k,
 *     b, lo32 step, hi32 step)); out = arg_{k*}.  Equal to flat sampling in
 *     distribution (hierarchical factorization).
 *   FS_COMBINE_MAX: k* = argmax_k pmax_k; out = arg_{k*}.  Equal to the flat
 *     sample exactly.
 *   Ties go to the lowest k; a row with no finite key gets -1.
 * Requires 1 <= n_groups <= 4096 and 1 <= B. */
int fs_group_combine(fs_ctx* ctx, void* stream, const fs_group_summary_t* s, int n_groups, int B, uint64_t seed,
                     uint64_t step, int mode, int32_t* out_idx);

/* Allocation-free variant of fs_fmms_sample, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It needs no context and calls no allocating routine:
 * the per-tile winners go to a static device array of this library (512 KiB
 * on each GPU it runs on, held until the process ends), whose device address
 * is looked up once per GPU (by fs_create on its device, else by this call's
 * first use on the current device).  The caller passes inputs and outputs as
 * for fs_fmms_sample, on the current HIP device:
 *   H [B, d], W [V, d] bf16 (row strides ldh, ldw), temperature, seed, step,
 *   mask (NULL or [B, ldm] words), out_idx [B] int32 device.
 * Same result as fs_fmms_sample with top_k = 0, no tile maxima and
 * FS_PATH_AUTO (same kernels and tiling).
 * Limits: 1 <= B <= 256 (FS_ERR_CAPACITY above), V < 2^31, and the other
 * requirements of fs_fmms_sample.  No top-k, tile maxima or several samples.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (two streams, two threads)
 * race and must be serialized by the caller. */
int fs_fmms_sample_noalloc(void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B,
                           int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                           const uint32_t* mask, int64_t ldm, int32_t* out_idx);

/* Timing hook for measurement.  The next streaming call made on this context
 * records `before` on its stream right before its streaming (LM-head) kernel
 * and `after` right after it, ahead of the small tile reduction that
 * follows, then forgets both; with several batch chunks, `before` precedes the
 * first chunk's kernel and `after` follows the last one's.  Both are
 * hipEvent_t handles passed as void*, created by the caller (with timing
 * enabled) and owned by it; both NULL disarms.  The elapsed time between them
 * is the streaming kernel's duration as seen on that stream.
 * Returns FS_ERR_INVALID_ARG if exactly one of them is NULL. */
int fs_profile_next_launch(fs_ctx* ctx, void* before, void* after);

/* Test exports. */

/* r_out[i] (if not NULL) = Philox word driving vocab id v0 + i of row `row` at
 * (seed, step); g_out[i] (if not NULL) = its fp32 Gumbel noise.  n >= 0,
 * v0 >= 0, v0 + n <= 2^31. */
int fs_debug_philox(fs_ctx* ctx, void* stream, uint64_t seed, uint64_t step, int row, int64_t v0, int64_t n,
                    uint32_t* r_out, float* g_out);

/* g_out[i] = fp32 Gumbel noise of the 32-bit word r0 + i (r0 + n <= 2^32). */
int fs_debug_gumbel_bits(fs_ctx* ctx, void* stream, uint64_t r0, int64_t n, float* g_out);

/* Exhaustive device scan of the noise transform over all 2^32 words.
 * stats_out (device, 4 x uint64): [0] = count of non-finite values,
 * [1] = count of words r where g(r) < g(r - 1), [2] = bits of the minimum as
 * float in the low 32 bits, [3] = same for the maximum. */
int fs_debug_gumbel_scan(fs_ctx* ctx, void* stream, uint64_t* stats_out);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSAMPLING_H_ */
