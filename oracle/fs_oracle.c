/*
 * fs_oracle.c -- CPU oracle for FlashSampling's fused LM-head matmul + sample.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously correct CPU
 * definition of what the sampler computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, constant table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * What is computed, and where it is stated:
 *   - Sampling from softmax(logits) by adding i.i.d. standard Gumbel noise to
 *     every logit and taking the argmax (the Gumbel-Max trick, "Theorem 2.1").
 *     [readus.org FlashSampling summary, section "Gumbel Max Trick"]
 *   - Logits are the LM-head product of hidden states and weights; the fused
 *     method computes them tile by tile, keeps one maximizer per row and per
 *     vocabulary tile and reduces over tiles; exact because argmax decomposes
 *     over a partition.  [FlashSampling, arXiv 2603.15854, abstract]
 *   - Grouped variants are exact by hierarchical factorization of the
 *     categorical; per group a log-sum-exp "captain" is kept, Gumbel noise on
 *     the captains picks the group, then a token is drawn inside it.
 *     [arXiv 2603.15854 abstract; readus.org summary, section "Group Gumbel Max"]
 *   - Forbidden ids are set to -inf before noise; top-k keeps a candidate set
 *     and runs exact Gumbel-Max inside it.
 *     [readus.org summary, section on Top-K and masking]
 *   - Noise comes from a Philox counter generator keyed by a master seed and
 *     the element's coordinates; the uniform is u = (r+1)/(2^32+1) for a 32-bit
 *     Philox word r, and the noise is -log(-log u).
 *     [readus.org summary, code guide sections 2 (RNG) and 3 (floating point)]
 *   - The API takes a temperature.  [readus.org summary, code guide section 1]
 *
 * Readings where the pages leave a step open (each is listed with its reason in
 * the design notes of this repository):
 *   R1  noise is keyed on the logical coordinates (seed, step, row, vocab id):
 *       Philox4x32-10 with key = (lo32(seed), hi32(seed)) and counter =
 *       (v >> 2, row, lo32(step), hi32(step)); the 32-bit word used for vocab
 *       id v is output word (v & 3).
 *   R2  temperature: s = logit / T in fp32; noise is added after scaling.
 *   R3  u is taken at its real-number value.  E = -ln u is evaluated without
 *       cancellation (log1p of -(1-u) when u > 1/2) in fp64; g = -ln E in fp64,
 *       then rounded once to fp32.
 *   R4  perturbed score p = s + g in fp32; argmax over fp32 p; ties go to the
 *       lowest vocab id; a row whose every p is -inf samples -1.
 *   R5  mask: uint32 words, bit (v & 31) of word (v >> 5) of the row, 1 means
 *       allowed.  Masking is applied before top-k.
 *   R6  top-k: the k largest s among allowed ids, ties at the boundary broken
 *       by lower id; all other ids get -inf.  Noise is the per-id noise of R1.
 *   R7  logits: every bf16 product is exact in fp64; products are summed in
 *       fp64 (ascending k) and the sum is rounded once to fp32.
 *   R8  grouped combine, mode G: group noise is the Gumbel transform of word 0
 *       of Philox(key = seed, counter = (0x40000000 | k, row, step)), a counter
 *       range the vocabulary never reaches; k* = argmax_k (lse_k + g'_k), the
 *       sample is that group's own argmax.  Mode M: k* = argmax_k pmax_k,
 *       which reproduces the flat argmax exactly.
 *   R10 top-p (nucleus) sampling, which two pages call compatible with the
 *       method without giving one, follows top-k: among the kept ids, sorted by
 *       score (descending, lower id first), the weights w = exp(s - s_max) are
 *       summed in fp64 in that order, and an id is kept while the weight of
 *       the ids before it is below top_p times their total (the shortest
 *       prefix whose mass reaches top_p of the kept mass).  top_p = 1 keeps
 *       every top-k id.  [nucleus sampling as defined by Holtzman et al., "The
 *       Curious Case of Neural Text Degeneration", ICLR 2020; cjcn.com.cn and
 *       news.neo-ai.one FlashSampling articles: compatible with top-p]
 *   R9  conventional comparator (not the method): one uniform per row and step
 *       from word 0 of Philox(key = seed, counter = (0x80000000, row, step)),
 *       u = (r+1)/(2^32+1); the sample is the first allowed id whose running
 *       sum of exp(s - max s) exceeds u times the total (fp64).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 storage: the upper 16 bits of an IEEE binary32.                     */
/* ------------------------------------------------------------------------ */
static float bf16_to_float(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, as defined by Salmon, Moraes, Dror and Shaw, "Parallel     */
/* Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds of a 4x32 Feistel-*/
/* like bijection driven by two 32x32->64 multiplications, with a Weyl       */
/* sequence added to the 2-word key between rounds.                          */
/* ------------------------------------------------------------------------ */
#define PHILOX_MUL_A 0xD2511F53u /* multiplies counter word 0 */
#define PHILOX_MUL_B 0xCD9E8D57u /* multiplies counter word 2 */
#define PHILOX_WEYL_0 0x9E3779B9u /* golden ratio */
#define PHILOX_WEYL_1 0xBB67AE85u /* sqrt(3) - 1 */

void fso_philox4x32_10(const uint32_t key[2], const uint32_t ctr[4], uint32_t out[4]) {
  uint32_t k0 = key[0], k1 = key[1];
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { /* key schedule: bump before every round but the first */
      k0 += PHILOX_WEYL_0;
      k1 += PHILOX_WEYL_1;
    }
    uint64_t prod_a = (uint64_t)PHILOX_MUL_A * (uint64_t)x0;
    uint64_t prod_b = (uint64_t)PHILOX_MUL_B * (uint64_t)x2;
    uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    uint32_t y0 = hi_b ^ x1 ^ k0;
    uint32_t y1 = lo_b;
    uint32_t y2 = hi_a ^ x3 ^ k1;
    uint32_t y3 = lo_a;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Reading R1: the Philox word that drives vocab id v of row `row` at `step`. */
uint32_t fso_noise_bits(uint64_t seed, uint64_t step, uint32_t row, uint32_t v) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {v >> 2, row, (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t out[4];
  fso_philox4x32_10(key, ctr, out);
  return out[v & 3u];
}

/* Reading R8: the Philox word for group k of row `row` (grouped mode G). */
uint32_t fso_group_noise_bits(uint64_t seed, uint64_t step, uint32_t row, uint32_t k) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {0x40000000u | k, row, (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t out[4];
  fso_philox4x32_10(key, ctr, out);
  return out[0];
}

/* Reading R9: the uniform of the conventional comparator's row `row` is
 * driven by word 0 of Philox(key = seed, counter = (0x80000000, row, step)),
 * a counter range that neither the vocabulary (v >> 2 < 2^29) nor the group
 * noise (0x40000000 | k, k < 2^30) reaches. */
uint32_t fso_uniform_bits(uint64_t seed, uint64_t step, uint32_t row) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {0x80000000u, row, (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t out[4];
  fso_philox4x32_10(key, ctr, out);
  return out[0];
}

/* u = (r + 1) / (2^32 + 1), strictly inside (0, 1), in fp64. */
double fso_uniform64(uint32_t r) { return ((double)r + 1.0) / 4294967297.0; }

/* ------------------------------------------------------------------------ */
/* Standard Gumbel noise from one 32-bit word (reading R3).                  */
/* u = (r + 1) / (2^32 + 1) lies strictly inside (0, 1).                    */
/* ------------------------------------------------------------------------ */
double fso_gumbel64(uint32_t r) {
  const double denom = 4294967297.0; /* 2^32 + 1, exact in binary64 */
  double e; /* e = -ln(u) > 0 */
  if (r < 2147483648u) {
    double u = ((double)r + 1.0) / denom; /* u <= 1/2: plain log is accurate */
    e = -log(u);
  } else {
    double one_minus_u = (4294967296.0 - (double)r) / denom; /* exact numerator */
    e = -log1p(-one_minus_u);
  }
  return -log(e);
}

float fso_gumbel32(uint32_t r) { return (float)fso_gumbel64(r); }

/* Fill out[i] = fp32 noise of word r0 + i, for i < n (wraps nothing: caller
 * keeps r0 + n <= 2^32). */
void fso_gumbel32_range(uint64_t r0, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = fso_gumbel32((uint32_t)(r0 + (uint64_t)i));
}

/* Scan words [r_lo, r_hi): count non-finite fp32 noise values and places
 * where the fp32 noise decreases from word r-1 to word r; report min and max.
 * stats = {nonfinite, decreases}; minmax = {min, max}. */
void fso_gumbel_scan(uint64_t r_lo, uint64_t r_hi, int64_t stats[2], double minmax[2]) {
  int64_t nonfinite = 0, decreases = 0;
  double mn = INFINITY, mx = -INFINITY;
#pragma omp parallel for schedule(static) reduction(+ : nonfinite, decreases) reduction(min : mn) reduction(max : mx)
  for (int64_t chunk = 0; chunk < 4096; ++chunk) {
    uint64_t span = r_hi - r_lo;
    uint64_t a = r_lo + span * (uint64_t)chunk / 4096u;
    uint64_t b = r_lo + span * (uint64_t)(chunk + 1) / 4096u;
    if (a >= b) continue;
    float prev = a > 0 ? fso_gumbel32((uint32_t)(a - 1)) : -INFINITY;
    for (uint64_t r = a; r < b; ++r) {
      float g = fso_gumbel32((uint32_t)r);
      if (!isfinite(g)) ++nonfinite;
      if (r > 0 && g < prev) ++decreases;
      if ((double)g < mn) mn = g;
      if ((double)g > mx) mx = g;
      prev = g;
    }
  }
  stats[0] = nonfinite;
  stats[1] = decreases;
  minmax[0] = mn;
  minmax[1] = mx;
}

/* ------------------------------------------------------------------------ */
/* Logits of the LM head: logits[b][v] = sum_k H[b][k] * W[v][k] (R7).       */
/* H is [B, d] with row stride ldh, W is [V, d] with row stride ldw, both    */
/* bf16 bit patterns.  Output is [B, V] fp32, row stride V.                   */
/* ------------------------------------------------------------------------ */
void fso_logits(const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B, int d,
                int64_t V, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int64_t v = 0; v < V; ++v) {
      const uint16_t* h = H + (int64_t)b * ldh;
      const uint16_t* w = W + v * ldw;
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += (double)bf16_to_float(h[k]) * (double)bf16_to_float(w[k]);
      out[(int64_t)b * V + v] = (float)acc;
    }
  }
}

/* Same product, fp32 accumulation in ascending k (used only by a test that
 * bounds the fp32-accumulation error of the kernels' arithmetic). */
void fso_logits_fp32acc(const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B, int d,
                        int64_t V, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int64_t v = 0; v < V; ++v) {
      const uint16_t* h = H + (int64_t)b * ldh;
      const uint16_t* w = W + v * ldw;
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc += bf16_to_float(h[k]) * bf16_to_float(w[k]);
      out[(int64_t)b * V + v] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Per-row sampling from precomputed logits.                                 */
/* ------------------------------------------------------------------------ */
static int mask_allows(const uint32_t* mask_row, int64_t v) {
  return (int)((mask_row[v >> 5] >> (uint32_t)(v & 31)) & 1u);
}

typedef struct {
  float s;
  int64_t id;
} scored_id;

/* Order for top-k: larger score first, equal scores by lower id (R6). */
static int by_score_desc_id_asc(const void* pa, const void* pb) {
  const scored_id* a = (const scored_id*)pa;
  const scored_id* b = (const scored_id*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Top-p within the ids a row keeps (R10): s holds V scores, -inf for ids
 * already excluded; ids past the nucleus are set to -inf. */
static void nucleus_filter(float* s, int64_t V, float top_p) {
  int64_t n = 0;
  for (int64_t v = 0; v < V; ++v)
    if (s[v] != -INFINITY && s[v] == s[v]) ++n;
  if (n == 0) return;
  scored_id* list = (scored_id*)malloc((size_t)n * sizeof(scored_id));
  int64_t i = 0;
  for (int64_t v = 0; v < V; ++v)
    if (s[v] != -INFINITY && s[v] == s[v]) {
      list[i].s = s[v];
      list[i].id = v;
      ++i;
    }
  qsort(list, (size_t)n, sizeof(scored_id), by_score_desc_id_asc);
  const double m = (double)list[0].s;
  double total = 0.0;
  for (i = 0; i < n; ++i) total += exp((double)list[i].s - m);
  double before = 0.0; /* weight of the ids ahead of list[i] */
  for (i = 0; i < n; ++i) {
    const double w = exp((double)list[i].s - m);
    if (!(before < (double)top_p * total)) s[list[i].id] = -INFINITY;
    before += w;
  }
  free(list);
}

/* Scaled, masked, top-k-filtered scores of one row (R2, R5, R6), then the
 * nucleus of the kept ids when top_p < 1 (R10).
 * s_out has V entries; excluded ids hold -inf. */
void fso_scores_row(const float* logit_row, int64_t V, float T, const uint32_t* mask_row, int top_k, float top_p,
                    float* s_out) {
  for (int64_t v = 0; v < V; ++v) {
    float s = logit_row[v] / T;
    if (mask_row && !mask_allows(mask_row, v)) s = -INFINITY;
    s_out[v] = s;
  }
  if (top_k > 0) {
    int64_t n_allowed = 0;
    for (int64_t v = 0; v < V; ++v)
      if (s_out[v] != -INFINITY) ++n_allowed;
    if (n_allowed > top_k) {
      scored_id* list = (scored_id*)malloc((size_t)n_allowed * sizeof(scored_id));
      int64_t n = 0;
      for (int64_t v = 0; v < V; ++v)
        if (s_out[v] != -INFINITY) {
          list[n].s = s_out[v];
          list[n].id = v;
          ++n;
        }
      qsort(list, (size_t)n, sizeof(scored_id), by_score_desc_id_asc);
      for (int64_t i = top_k; i < n; ++i) s_out[list[i].id] = -INFINITY;
      free(list);
    }
  }
  if (top_p < 1.0f) nucleus_filter(s_out, V, top_p);
}

/* Perturbed scores p = s + g of one row (R1, R4). */
void fso_perturbed_row(const float* logit_row, int64_t V, float T, uint64_t seed, uint64_t step, int row,
                       const uint32_t* mask_row, int top_k, float top_p, float* p_out) {
  fso_scores_row(logit_row, V, T, mask_row, top_k, top_p, p_out);
  for (int64_t v = 0; v < V; ++v) {
    float g = fso_gumbel32(fso_noise_bits(seed, step, (uint32_t)row, (uint32_t)v));
    p_out[v] = p_out[v] + g; /* -inf stays -inf */
  }
}

/* Argmax with the lowest-id tie rule; -1 if every entry is -inf (or NaN). */
int64_t fso_argmax(const float* p, int64_t n) {
  float best = -INFINITY;
  int64_t arg = -1;
  for (int64_t i = 0; i < n; ++i)
    if (p[i] > best) {
      best = p[i];
      arg = i;
    }
  return arg;
}

/* One sampling step for B rows from logits [B, V] (row stride V).
 * mask: NULL or [B, ldm] words.  p_out: NULL or [B, V] perturbed scores. */
void fso_sample_from_logits(const float* logits, int B, int64_t V, float T, uint64_t seed, uint64_t step,
                            const uint32_t* mask, int64_t ldm, int top_k, float top_p, int32_t* out_idx,
                            float* p_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    float* p = p_out ? p_out + (int64_t)b * V : (float*)malloc((size_t)V * sizeof(float));
    fso_perturbed_row(logits + (int64_t)b * V, V, T, seed, step, b, mask ? mask + (int64_t)b * ldm : NULL,
                      top_k, top_p, p);
    out_idx[b] = (int32_t)fso_argmax(p, V);
    if (!p_out) free(p);
  }
}

/* Conventional comparator (not the method): sample one row by inverse CDF.
 * Scores as R2 and R5 (mask, no top-k); weights w_v = exp(s_v - m) in fp64
 * over the allowed ids, m their largest score; Z = sum of w; the sample is
 * the first id whose running sum of w exceeds u * Z (the last allowed id if
 * rounding leaves the sum at or below it); -1 if no id is allowed.  This is
 * the softmax, prefix-sum and search pipeline that the fused sampler replaces.
 * [readus.org FlashSampling summary, the essay part: the softmax pipeline
 * exponentiates, normalizes and scans a cumulative array to pick a token] */
int64_t fso_cdf_sample_row(const float* logit_row, int64_t V, float T, const uint32_t* mask_row, double u) {
  float* s = (float*)malloc((size_t)V * sizeof(float));
  fso_scores_row(logit_row, V, T, mask_row, 0, 1.0f, s);
  double m = -INFINITY;
  int64_t last = -1;
  for (int64_t v = 0; v < V; ++v)
    if (s[v] != -INFINITY) {
      if ((double)s[v] > m) m = (double)s[v];
      last = v;
    }
  int64_t pick = last;
  if (last >= 0) {
    double Z = 0.0;
    for (int64_t v = 0; v < V; ++v)
      if (s[v] != -INFINITY) Z += exp((double)s[v] - m);
    const double target = u * Z;
    double run = 0.0;
    for (int64_t v = 0; v < V; ++v) {
      if (s[v] == -INFINITY) continue;
      run += exp((double)s[v] - m);
      if (run > target) {
        pick = v;
        break;
      }
    }
  }
  free(s);
  return pick;
}

/* The comparator over steps step0 .. step0+nsteps-1 of global rows `rows`
 * (logits[i] belongs to row rows[i]); out is [nsteps, R]; u_out, if not NULL,
 * receives the uniforms. */
void fso_cdf_sample_rows_steps(const float* logits, const int32_t* rows, int R, int64_t V, float T, uint64_t seed,
                               uint64_t step0, int nsteps, const uint32_t* mask, int64_t ldm, int32_t* out,
                               double* u_out) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int t = 0; t < nsteps; ++t)
    for (int i = 0; i < R; ++i) {
      const double u = fso_uniform64(fso_uniform_bits(seed, step0 + (uint64_t)t, (uint32_t)rows[i]));
      if (u_out) u_out[(int64_t)t * R + i] = u;
      out[(int64_t)t * R + i] = (int32_t)fso_cdf_sample_row(logits + (int64_t)i * V, V, T,
                                                            mask ? mask + (int64_t)rows[i] * ldm : NULL, u);
    }
}

/* Many consecutive steps step0 .. step0+nsteps-1 for fixed logits; out is
 * [nsteps, B].  Used by the distributional tests. */
void fso_sample_steps(const float* logits, int B, int64_t V, float T, uint64_t seed, uint64_t step0,
                      int64_t nsteps, const uint32_t* mask, int64_t ldm, int top_k, float top_p, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < nsteps; ++t) {
    float* p = (float*)malloc((size_t)V * sizeof(float));
    for (int b = 0; b < B; ++b) {
      fso_perturbed_row(logits + (int64_t)b * V, V, T, seed, step0 + (uint64_t)t, b,
                        mask ? mask + (int64_t)b * ldm : NULL, top_k, top_p, p);
      out[t * B + b] = (int32_t)fso_argmax(p, V);
    }
    free(p);
  }
}

/* Samples of selected rows over steps step0 .. step0+nsteps-1.  logits is
 * [R, V] holding the logits of global batch rows rows[0..R-1]; the noise and
 * the mask row use the global row id.  out_idx and out_pmax are [nsteps, R]:
 * the sampled id and its perturbed score. */
void fso_sample_rows_steps(const float* logits, const int32_t* rows, int R, int64_t V, float T, uint64_t seed,
                           uint64_t step0, int64_t nsteps, const uint32_t* mask, int64_t ldm, int top_k,
                           float top_p, int32_t* out_idx, float* out_pmax) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t t = 0; t < nsteps; ++t) {
    for (int i = 0; i < R; ++i) {
      float* p = (float*)malloc((size_t)V * sizeof(float));
      fso_perturbed_row(logits + (int64_t)i * V, V, T, seed, step0 + (uint64_t)t, rows[i],
                        mask ? mask + (int64_t)rows[i] * ldm : NULL, top_k, top_p, p);
      int64_t a = fso_argmax(p, V);
      out_idx[t * R + i] = (int32_t)a;
      out_pmax[t * R + i] = a < 0 ? -INFINITY : p[a];
      free(p);
    }
  }
}

/* Per-tile maxima of perturbed scores for one step: tiles are the vocab
 * ranges [bounds[i], bounds[i+1]).  Outputs are [B, n_tiles]. */
void fso_tile_maxima(const float* logits, int B, int64_t V, float T, uint64_t seed, uint64_t step,
                     const uint32_t* mask, int64_t ldm, const int64_t* bounds, int n_tiles, float* tile_max,
                     int32_t* tile_arg) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    float* p = (float*)malloc((size_t)V * sizeof(float));
    fso_perturbed_row(logits + (int64_t)b * V, V, T, seed, step, b, mask ? mask + (int64_t)b * ldm : NULL, 0,
                      1.0f, p);
    for (int i = 0; i < n_tiles; ++i) {
      int64_t lo = bounds[i], hi = bounds[i + 1];
      int64_t a = fso_argmax(p + lo, hi - lo);
      tile_max[(int64_t)b * n_tiles + i] = a < 0 ? -INFINITY : p[lo + a];
      tile_arg[(int64_t)b * n_tiles + i] = a < 0 ? -1 : (int32_t)(lo + a);
    }
    free(p);
  }
}

/* ------------------------------------------------------------------------ */
/* Grouped (online) variant.                                                 */
/* ------------------------------------------------------------------------ */

/* Summary of one vocabulary group [lo, hi) of one row from its scores s and
 * perturbed scores p: lse = log sum exp(s) over allowed ids (fp64, rounded to
 * fp32; -inf if none), and the group's perturbed maximum and its id. */
static void group_summary_row(const float* s, const float* p, int64_t lo, int64_t hi, float* lse, float* pmax,
                              int32_t* arg) {
  double m = -INFINITY;
  for (int64_t v = lo; v < hi; ++v)
    if ((double)s[v] > m) m = s[v];
  if (m == -INFINITY) {
    *lse = -INFINITY;
  } else {
    double acc = 0.0;
    for (int64_t v = lo; v < hi; ++v)
      if (s[v] != -INFINITY) acc += exp((double)s[v] - m);
    *lse = (float)(m + log(acc));
  }
  int64_t a = fso_argmax(p + lo, hi - lo);
  *pmax = a < 0 ? -INFINITY : p[lo + a];
  *arg = a < 0 ? -1 : (int32_t)(lo + a);
}

/* Summaries of group [vocab_offset, vocab_offset + G) for B rows.  logits is
 * [B, V_total] (row stride V_total); vocab ids are global, so the noise is the
 * flat noise.  Outputs lse, pmax, arg are [B]. */
void fso_group_summary(const float* logits, int B, int64_t V_total, int64_t vocab_offset, int64_t G, float T,
                       uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm, float* lse, float* pmax,
                       int32_t* arg) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    float* s = (float*)malloc((size_t)V_total * sizeof(float));
    float* p = (float*)malloc((size_t)V_total * sizeof(float));
    const float* row = logits + (int64_t)b * V_total;
    const uint32_t* mrow = mask ? mask + (int64_t)b * ldm : NULL;
    for (int64_t v = vocab_offset; v < vocab_offset + G; ++v) {
      float sv = row[v] / T;
      if (mrow && !mask_allows(mrow, v)) sv = -INFINITY;
      s[v] = sv;
      p[v] = sv + fso_gumbel32(fso_noise_bits(seed, step, (uint32_t)b, (uint32_t)v));
    }
    group_summary_row(s, p, vocab_offset, vocab_offset + G, &lse[b], &pmax[b], &arg[b]);
    free(s);
    free(p);
  }
}

/* Combine n_groups summaries ([n_groups, B] each) into one sample per row.
 * mode 0 (G): hierarchical Group-Gumbel-Max (R8).  mode 1 (M): max of the
 * perturbed maxima.  Ties go to the lowest group; a row with no finite
 * candidate samples -1. */
void fso_group_combine(const float* lse, const float* pmax, const int32_t* arg, int n_groups, int B,
                       uint64_t seed, uint64_t step, int mode, int32_t* out_idx) {
  for (int b = 0; b < B; ++b) {
    float best = -INFINITY;
    int kbest = -1;
    for (int k = 0; k < n_groups; ++k) {
      float key;
      if (mode == 0)
        key = lse[(int64_t)k * B + b] + fso_gumbel32(fso_group_noise_bits(seed, step, (uint32_t)b, (uint32_t)k));
      else
        key = pmax[(int64_t)k * B + b];
      if (key > best) {
        best = key;
        kbest = k;
      }
    }
    out_idx[b] = kbest < 0 ? -1 : arg[(int64_t)kbest * B + b];
  }
}

/* Grouped sampling over many steps for fixed logits, groups given by bounds
 * [n_groups + 1] over [0, V).  out is [nsteps, B].  Used by the tests that
 * compare grouped and flat sampling in distribution. */
void fso_grouped_sample_steps(const float* logits, int B, int64_t V, float T, uint64_t seed, uint64_t step0,
                              int64_t nsteps, const uint32_t* mask, int64_t ldm, const int64_t* bounds,
                              int n_groups, int mode, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < nsteps; ++t) {
    uint64_t step = step0 + (uint64_t)t;
    float* s = (float*)malloc((size_t)V * sizeof(float));
    float* p = (float*)malloc((size_t)V * sizeof(float));
    float* lse = (float*)malloc((size_t)n_groups * (size_t)B * sizeof(float));
    float* pmax = (float*)malloc((size_t)n_groups * (size_t)B * sizeof(float));
    int32_t* arg = (int32_t*)malloc((size_t)n_groups * (size_t)B * sizeof(int32_t));
    for (int b = 0; b < B; ++b) {
      const uint32_t* mrow = mask ? mask + (int64_t)b * ldm : NULL;
      fso_scores_row(logits + (int64_t)b * V, V, T, mrow, 0, 1.0f, s);
      for (int64_t v = 0; v < V; ++v) p[v] = s[v] + fso_gumbel32(fso_noise_bits(seed, step, (uint32_t)b, (uint32_t)v));
      for (int k = 0; k < n_groups; ++k)
        group_summary_row(s, p, bounds[k], bounds[k + 1], &lse[(int64_t)k * B + b], &pmax[(int64_t)k * B + b],
                          &arg[(int64_t)k * B + b]);
    }
    fso_group_combine(lse, pmax, arg, n_groups, B, seed, step, mode, out + t * B);
    free(s);
    free(p);
    free(lse);
    free(pmax);
    free(arg);
  }
}

/* ------------------------------------------------------------------------ */
/* End to end, from bf16 operands: the whole fused sampler's definition.     */
/* ------------------------------------------------------------------------ */
void fso_fmms_sample(const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B, int d, int64_t V,
                     float T, uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm, int top_k,
                     float top_p, int32_t* out_idx) {
  float* logits = (float*)malloc((size_t)B * (size_t)V * sizeof(float));
  fso_logits(H, ldh, W, ldw, B, d, V, logits);
  fso_sample_from_logits(logits, B, V, T, seed, step, mask, ldm, top_k, top_p, out_idx, NULL);
  free(logits);
}

int fso_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
