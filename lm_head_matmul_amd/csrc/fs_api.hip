// fs_api.hip -- C ABI of the FlashSampling library: argument checks, the
// per-context device workspace, kernel selection and launches.  Every entry
// point validates synchronously, enqueues on the caller's stream and returns.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/flashsampling.h"
#include "fs_kernels.h"

struct fs_ctx {
  int device;
  int max_B;
  int64_t max_V;
  int max_top_k;
  int n_cu;
  int max_tiles;
  // [max_B][max_tiles] per-tile winners (and log-sum-exp state)
  float* ws_val;
  int32_t* ws_idx;
  float* ws_m;
  float* ws_s;
  void* base;
  // fused top-k: per (row, tile) candidate lists of up to topk_rows rows
  uint64_t* topk_lists;
  // top-k from stored scores (k above kTopkFusedMax, the dot path, and the
  // unfused comparator): fp32 scores of up to topk_rows batch rows,
  // [topk_rows][topk_ldl] (allocated when max_top_k > kTopkFusedMax)
  float* topk_ws;
  int64_t topk_ldl;
  int topk_rows;
  // top-k selection workspace for topk_rows rows (see fsk::TopkParams)
  void* topk_sel;
  uint32_t* topk_hist;
  uint64_t* topk_cand;
  int32_t* topk_cand_n;
  float* topk_seg_val;
  int32_t* topk_seg_idx;
  int32_t* topk_bound;
  uint32_t* topk_arrive;
  // conventional comparator: [max_B][kCdfMaxSeg] segment max, sum of exp, sum of probabilities
  float* cdf_ws;
  // timing hook (fs_profile_next_launch): events the next streaming call records
  hipEvent_t prof_before;
  hipEvent_t prof_after;
};

namespace {

// A fixed buffer: reporting an error allocates nothing.
thread_local char g_error[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Runs the call with ctx->device current and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      ok = false;
      return;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : dflt;
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Kernel choice for a batch chunk of `B` rows (B <= kMfmaMaxB, or <= kWideMaxB for the wide kernel,
// whose chunks run_stream_chunks forms only where that kernel applies).
int choose_config(int B, int path, fsk::StreamConfig& cfg) {
  // AUTO takes the MFMA kernel at every batch size: on gfx950 it streams W
  // faster than the dot-product kernel even at B = 1 (measured).
  const int dot_max = env_int("FS_DOT_MAX_B", 0);
  bool dot;
  if (path == FS_PATH_DOT) {
    if (B > fsk::kDotMaxB) return fail(FS_ERR_UNSUPPORTED, "dot-product path supports B <= %d (got %d)", fsk::kDotMaxB, B);
    dot = true;
  } else if (path == FS_PATH_MFMA) {
    dot = false;
  } else {
    dot = B <= dot_max && B <= fsk::kDotMaxB;
  }
  cfg.dot = dot;
  cfg.bd = dot ? pow2_at_least(B) : 0;
  cfg.nb = dot ? 0 : (B <= 16 ? 1 : B <= 32 ? 2 : B <= fsk::kMfmaMaxB ? 4 : fsk::wide_nb(B));
  cfg.fast = false;
  cfg.rm = 0;
  cfg.lds_bytes = 0;
  return FS_OK;
}

int64_t mask_words(int64_t V) { return (V + 31) / 32; }

int n_tiles_for(const fs_ctx* ctx, int64_t V) {
  const int64_t nmb = (V + 15) / 16;
  return (int)(nmb < ctx->max_tiles ? nmb : ctx->max_tiles);
}

// Common checks of the operands of a streaming call.
int check_operands(const fs_ctx* ctx, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B, int d,
                   int64_t V, float temperature, const uint32_t* mask, int64_t ldm, int64_t mask_V) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (!H || !W) return fail(FS_ERR_INVALID_ARG, "H and W must be non-NULL device pointers");
  if (B < 1 || B > ctx->max_B) return fail(B < 1 ? FS_ERR_INVALID_ARG : FS_ERR_CAPACITY, "B=%d outside [1, max_B=%d]", B, ctx->max_B);
  if (d < 8 || d % 8 != 0) return fail(FS_ERR_INVALID_ARG, "d=%d must be a positive multiple of 8", d);
  if (ldh < d || ldh % 8 != 0) return fail(FS_ERR_INVALID_ARG, "ldh=%lld must be >= d and a multiple of 8", (long long)ldh);
  if (ldw < d || ldw % 8 != 0) return fail(FS_ERR_INVALID_ARG, "ldw=%lld must be >= d and a multiple of 8", (long long)ldw);
  if (!aligned16(H) || !aligned16(W)) return fail(FS_ERR_INVALID_ARG, "H and W must be 16-byte aligned");
  if (V < 1) return fail(FS_ERR_INVALID_ARG, "V=%lld must be >= 1", (long long)V);
  if (V > ctx->max_V) return fail(FS_ERR_CAPACITY, "V=%lld exceeds max_V=%lld", (long long)V, (long long)ctx->max_V);
  if (!(std::isfinite(temperature) && temperature > 0.0f))
    return fail(FS_ERR_INVALID_ARG, "temperature must be finite and > 0 (got %g)", (double)temperature);
  if (mask && ldm < mask_words(mask_V))
    return fail(FS_ERR_INVALID_ARG, "ldm=%lld must be >= ceil(V/32)=%lld", (long long)ldm, (long long)mask_words(mask_V));
  return FS_OK;
}

// Fills the fields common to all streaming launches.
void fill_common(fsk::StreamParams& p, const fs_ctx* ctx, const uint16_t* H, int64_t ldh, const uint16_t* W,
                 int64_t ldw, int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                 const uint32_t* mask, int64_t ldm) {
  std::memset(&p, 0, sizeof p);
  p.H = H;
  p.ldh = ldh;
  p.W = W;
  p.ldw = ldw;
  p.B = B;
  p.d = d;
  p.V = V;
  p.inv_t = 1.0f / temperature;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  p.step_lo = (uint32_t)step;
  p.step_hi = (uint32_t)(step >> 32);
  p.mask = mask;
  p.ldm = ldm;
  p.n_tiles = n_tiles_for(ctx, V);
  p.n_mblocks = (V + 15) / 16;
  p.ws_val = ctx->ws_val;
  p.ws_idx = ctx->ws_idx;
  p.ws_m = ctx->ws_m;
  p.ws_s = ctx->ws_s;
  p.top_p = 1.0f;
}

// Launches the streaming kernel over the batch in chunks of at most
// kMfmaMaxB rows, or kWideMaxB rows for the wide kernel when `wide` allows it
// (each chunk streams W once); with a mask, chunks are also small enough for
// their tile masks to fit the LDS staging area.  `per_chunk`
// adjusts the output pointers of a chunk that starts at batch row r0.
// With base.samples > 1, base.B counts the call's virtual rows (row h, sample
// s at h * samples + s): H and row_offset stay those of the call and each chunk
// starts at virtual row r0; `max_rows` bounds a chunk by the context's workspace.
// Events armed by fs_profile_next_launch are recorded before the first chunk's
// streaming kernel and after the last one's, then disarmed.
template <typename F>
int run_stream_chunks(fs_ctx* ctx, fsk::StreamParams base, int path, int epi, hipStream_t stream, F per_chunk,
                      int max_rows = fsk::kMfmaMaxB, bool wide = false) {
  const int B = base.B;
  hipEvent_t ev_before = ctx->prof_before, ev_after = ctx->prof_after;
  ctx->prof_before = ctx->prof_after = nullptr;
  int chunk = fsk::kMfmaMaxB < max_rows ? fsk::kMfmaMaxB : max_rows;
  // more than kMfmaMaxB rows of the plain sampler: chunks of kWideMaxB rows for
  // the wide kernel, which streams W once per chunk (any chunk of 65 .. 256
  // rows, the last one included, needs d to be a multiple of both its k rings)
  if (wide && B > fsk::kMfmaMaxB && max_rows >= fsk::kWideMaxB && path != FS_PATH_DOT && !base.mask &&
      base.samples <= 1 && base.d % fsk::wide_kmult(8) == 0 && base.d % fsk::wide_kmult(16) == 0 &&
      epi == fsk::EPI_FLAT)
    chunk = fsk::kWideMaxB;
  if (base.mask) {
    const int64_t rows = fsk::kMaskLdsMax / (4 * fsk::tile_mask_words(base.n_mblocks, base.n_tiles));
    if (rows < 1) return fail(FS_ERR_UNSUPPORTED, "V=%lld: a tile's mask does not fit the LDS staging area", (long long)base.V);
    if (rows < chunk) chunk = (int)rows;
  }
  for (int r0 = 0; r0 < B; r0 += chunk) {
    const int Bc = (B - r0) < chunk ? (B - r0) : chunk;
    fsk::StreamParams p = base;
    p.B = Bc;
    if (base.samples > 1) {
      p.vrow0 = r0;
    } else {
      p.H = base.H + (int64_t)r0 * base.ldh;
      p.row_offset = r0;
    }
    per_chunk(p, r0);
    fsk::StreamConfig cfg;
    int rc = choose_config(Bc, path, cfg);
    if (rc != FS_OK) return rc;
    if (!fsk::plan_stream(p, cfg, epi))
      return fail(FS_ERR_UNSUPPORTED, "shape B=%d d=%d does not fit the LDS budget", Bc, p.d);
    const bool last = r0 + chunk >= B;
    hipError_t e = fsk::launch_stream(p, cfg, epi, stream, r0 == 0 ? ev_before : nullptr, last ? ev_after : nullptr);
    if (e != hipSuccess) return hip_fail(e, "streaming kernel launch");
  }
  return FS_OK;
}

// Top-k sampling of batch rows [r0, r0 + rows) whose unscaled logits are in
// logits (row r0 first).
int launch_topk(const fs_ctx* ctx, const float* logits, int64_t ldl, int rows, int r0, int64_t V, float temperature,
                uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm, int top_k, int32_t* out_idx,
                hipStream_t s) {
  fsk::TopkParams q;
  std::memset(&q, 0, sizeof q);
  q.ldl = ldl;
  q.V = (int)V;
  q.inv_t = 1.0f / temperature;
  q.seed_lo = (uint32_t)seed;
  q.seed_hi = (uint32_t)(seed >> 32);
  q.step_lo = (uint32_t)step;
  q.step_hi = (uint32_t)(step >> 32);
  q.mask = mask;
  q.ldm = ldm;
  q.top_k = top_k;
  q.hist = ctx->topk_hist;
  q.cand = ctx->topk_cand;
  q.cand_n = ctx->topk_cand_n;
  q.seg_val = ctx->topk_seg_val;
  q.seg_idx = ctx->topk_seg_idx;
  q.bound = ctx->topk_bound;
  q.arrive_hist = ctx->topk_arrive;
  q.arrive_coll = ctx->topk_arrive + ctx->topk_rows;
  // rows are processed in chunks of the workspace's topk_rows; each row is split
  // into segments so that a chunk launches about 512 workgroups, with segments
  // of at least 2048 quads: each workgroup's fixed latency (a device-scope
  // round trip to count its arrival) then weighs less than its stretch of the
  // scores (measured best on MI355X at 1 to 64 rows of 151936 scores)
  for (int c0 = 0; c0 < rows; c0 += ctx->topk_rows) {
    const int n = (rows - c0) < ctx->topk_rows ? (rows - c0) : ctx->topk_rows;
    const int64_t nq = (V + 3) / 4;
    int64_t seg = 512 / n;
    if (seg > nq / 2048) seg = nq / 2048;
    if (seg > fsk::kTopkMaxSeg) seg = fsk::kTopkMaxSeg;
    if (seg < 1) seg = 1;
    q.logits = logits + (int64_t)c0 * ldl;
    q.B = n;
    q.row_offset = r0 + c0;
    q.out_idx = out_idx + r0 + c0;
    q.n_seg = (int)seg;
    hipError_t e = fsk::launch_topk_sample(q, s);
    if (e != hipSuccess) return hip_fail(e, "top-k sampling kernel launch");
  }
  return FS_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free sampling (fs_fmms_sample_noalloc).  Its per-tile winners --
// the only device memory the plain sampler needs beyond the caller's inputs
// and outputs -- live in one file-scope device array instead of a context's
// workspace: [kNoAllocMaxB][kNoAllocMaxTiles] fp32 values, then as many int32
// ids.  Each GPU holds its own copy of the array until the process ends.  In
// host code `scratch` only names the symbol; its device address on each GPU
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr int kNoAllocMaxB = 256;
constexpr int kNoAllocMaxTiles = 256;
constexpr size_t kNoAllocScratchBytes = (size_t)kNoAllocMaxB * kNoAllocMaxTiles * 8;  // 512 KiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
struct NoAllocDevice {
  unsigned char* ptr;  // device address of this GPU's copy of `scratch` (null: not set up yet)
  int n_cu;
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kNoAllocMaxDevices];

// Looks up (once per device) the address of the device's `scratch`; `dev` must be current.
int noalloc_setup(int dev, NoAllocDevice& out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(FS_ERR_UNSUPPORTED, "device %d: the allocation-free path supports devices 0..%d", dev,
                kNoAllocMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoAllocDevice& d = g_noalloc[dev];
  if (d.ptr == nullptr) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(FS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    int n_cu = 0;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    d.n_cu = n_cu;
    d.ptr = (unsigned char*)ptr;
  }
  out = d;
  return FS_OK;
}

// Fused top-k (and its nucleus): the streaming pass keeps short candidate
// lists per (row, tile) instead of the scores, and a merge launch per
// batch chunk selects the top k, cuts the nucleus when top_p < 1, and samples.
int sample_topk_fused(fs_ctx* ctx, hipStream_t stream, const uint16_t* H, int64_t ldh, const uint16_t* W,
                      int64_t ldw, int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                      const uint32_t* mask, int64_t ldm, int top_k, float top_p, int32_t* out_idx, int path) {
  fsk::StreamParams p;
  fill_common(p, ctx, H, ldh, W, ldw, B, d, V, temperature, seed, step, mask, ldm);
  p.top_k = top_k;
  p.top_p = top_p;
  p.topk_cand = ctx->topk_lists;
  return run_stream_chunks(
      ctx, p, path, fsk::EPI_TOPK, stream,
      [&](fsk::StreamParams& c, int r0) {
        c.out_idx = out_idx + r0;
        c.tile_ratio = mask ? 0 : fsk::kXcdTileRatio;
      },
      ctx->topk_rows);
}

}  // namespace

extern "C" {

const char* fs_last_error(void) { return g_error; }

int fs_create(fs_ctx** out, int device, int max_B, int64_t max_V, int max_top_k) {
  if (!out) return fail(FS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (max_B < 1) return fail(FS_ERR_INVALID_ARG, "max_B=%d must be >= 1", max_B);
  if (max_V < 1 || max_V >= ((int64_t)1 << 31)) return fail(FS_ERR_INVALID_ARG, "max_V must be in [1, 2^31)");
  if (max_top_k < 0) return fail(FS_ERR_INVALID_ARG, "max_top_k must be >= 0");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(FS_ERR_INVALID_ARG, "device %d outside [0, %d)", device, ndev);
  DeviceGuard guard(device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", device);
  fs_ctx* c = new fs_ctx();
  std::memset(c, 0, sizeof *c);
  c->device = device;
  c->max_B = max_B;
  c->max_V = max_V;
  c->max_top_k = max_top_k;
  e = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  // one vocabulary tile per CU; the fused top-k's merge holds a tile per thread
  c->max_tiles = c->n_cu < fsk::kTopkMergeThreads ? c->n_cu : fsk::kTopkMergeThreads;
  {  // the allocation-free entry point's scratch address on this device, looked up at set-up
    NoAllocDevice nd;
    const int rc = noalloc_setup(device, nd);
    if (rc != FS_OK) {
      delete c;
      return rc;
    }
  }
  const size_t n = (size_t)max_B * (size_t)c->max_tiles;
  const size_t bytes = 4 * n * sizeof(float) + 256;
  e = hipMalloc(&c->base, bytes);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipMalloc(workspace)");
  }
  char* b = (char*)c->base;
  c->ws_val = (float*)b;
  c->ws_idx = (int32_t*)(c->ws_val + n);
  c->ws_m = (float*)(c->ws_idx + n);
  c->ws_s = c->ws_m + n;
  e = hipMemset(c->base, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(c->base);
    delete c;
    return hip_fail(e, "hipMemset(workspace)");
  }
  e = hipMalloc(&c->cdf_ws, (size_t)3 * max_B * fsk::kCdfMaxSeg * sizeof(float));
  if (e != hipSuccess) {
    (void)hipFree(c->base);
    delete c;
    return hip_fail(e, "hipMalloc(comparator workspace)");
  }
  if (max_top_k > 0) {
    c->topk_rows = max_B < fsk::kMfmaMaxB ? max_B : fsk::kMfmaMaxB;
    c->topk_ldl = (max_V + 3) / 4 * 4;
    const size_t lists = (size_t)c->topk_rows * c->max_tiles * fsk::kTopkSlot * sizeof(uint64_t);
    e = hipMalloc(&c->topk_lists, lists);
    if (e == hipSuccess && max_top_k > fsk::kTopkFusedMax)
      e = hipMalloc(&c->topk_ws, (size_t)c->topk_rows * (size_t)c->topk_ldl * sizeof(float));
    if (e != hipSuccess) {
      if (c->topk_lists) (void)hipFree(c->topk_lists);
      (void)hipFree(c->cdf_ws);
      (void)hipFree(c->base);
      delete c;
      return hip_fail(e, "hipMalloc(top-k workspace)");
    }
    // selection workspace: cand [rows][cap] u64, hist [rows][bins] u32, seg_val / seg_idx
    // [rows][max_seg], cand_n [rows], bound [rows][4], two arrival counters [rows];
    // hist, cand_n and the counters start at zero and every call leaves them at zero
    const size_t R = (size_t)c->topk_rows;
    const size_t sel =
        R * fsk::kTopkCap * 8 + R * fsk::kTopkBins * 4 + R * fsk::kTopkMaxSeg * 8 + R * 4 + R * 16 + R * 8;
    e = hipMalloc(&c->topk_sel, sel);
    if (e == hipSuccess) e = hipMemset(c->topk_sel, 0, sel);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      if (c->topk_sel) (void)hipFree(c->topk_sel);
      if (c->topk_ws) (void)hipFree(c->topk_ws);
      (void)hipFree(c->topk_lists);
      (void)hipFree(c->cdf_ws);
      (void)hipFree(c->base);
      delete c;
      return hip_fail(e, "top-k selection workspace");
    }
    char* t = (char*)c->topk_sel;
    c->topk_cand = (uint64_t*)t;
    c->topk_hist = (uint32_t*)(t + R * fsk::kTopkCap * 8);
    c->topk_seg_val = (float*)(t + R * fsk::kTopkCap * 8 + R * fsk::kTopkBins * 4);
    c->topk_seg_idx = (int32_t*)(c->topk_seg_val + R * fsk::kTopkMaxSeg);
    c->topk_cand_n = (int32_t*)(c->topk_seg_idx + R * fsk::kTopkMaxSeg);
    c->topk_bound = c->topk_cand_n + R;
    c->topk_arrive = (uint32_t*)(c->topk_bound + 4 * R);
  }
  *out = c;
  return FS_OK;
}

void fs_destroy(fs_ctx* ctx) {
  if (!ctx) return;
  DeviceGuard guard(ctx->device);
  if (ctx->base) (void)hipFree(ctx->base);
  if (ctx->topk_ws) (void)hipFree(ctx->topk_ws);
  if (ctx->topk_lists) (void)hipFree(ctx->topk_lists);
  if (ctx->topk_sel) (void)hipFree(ctx->topk_sel);
  if (ctx->cdf_ws) (void)hipFree(ctx->cdf_ws);
  delete ctx;
}

int fs_fmms_tiling(fs_ctx* ctx, int B, int d, int64_t V, int path, int64_t* n_tiles, int64_t* bounds) {
  (void)d;
  (void)path;
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (B < 1 || V < 1 || V > ctx->max_V) return fail(FS_ERR_INVALID_ARG, "B or V out of range");
  const int nt = n_tiles_for(ctx, V);
  const int64_t nmb = (V + 15) / 16;
  if (n_tiles) *n_tiles = nt;
  if (bounds) {
    for (int i = 0; i <= nt; ++i) {
      const int64_t r = 16 * ((int64_t)i * nmb / nt);
      bounds[i] = r < V ? r : V;
    }
  }
  return FS_OK;
}

int fs_fmms_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B,
                   int d, int64_t V, float temperature, uint64_t seed, uint64_t step, const uint32_t* mask,
                   int64_t ldm, int top_k, int32_t* out_idx, float* tile_max, int32_t* tile_arg, int path) {
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, V, temperature, mask, ldm, V);
  if (rc != FS_OK) return rc;
  if (!out_idx) return fail(FS_ERR_INVALID_ARG, "out_idx is NULL");
  if (top_k < 0 || top_k > ctx->max_top_k)
    return fail(top_k < 0 ? FS_ERR_INVALID_ARG : FS_ERR_CAPACITY, "top_k=%d outside [0, max_top_k=%d]", top_k, ctx->max_top_k);
  if ((tile_max == nullptr) != (tile_arg == nullptr)) return fail(FS_ERR_INVALID_ARG, "tile_max and tile_arg go together");
  if (top_k > 0 && tile_max) return fail(FS_ERR_INVALID_ARG, "tile maxima are reported with top_k == 0 only");
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  fsk::StreamParams p;
  if (top_k > 0 && top_k <= fsk::kTopkFusedMax && path != FS_PATH_DOT)
    return sample_topk_fused(ctx, (hipStream_t)stream, H, ldh, W, ldw, B, d, V, temperature, seed, step, mask, ldm,
                             top_k, 1.0f, out_idx, path);
  if (top_k > 0) {
    // Larger k, or the dot-product path: the exact top-k boundary of a row is
    // found from all of its scores, which the streaming pass stores into the
    // context's workspace (batch chunks of topk_rows rows); the selection
    // launches sample the kept set.
    if (!ctx->topk_ws)
      return fail(FS_ERR_CAPACITY, "top_k=%d on this path needs a context created with max_top_k > %d", top_k,
                  fsk::kTopkFusedMax);
    hipStream_t s = (hipStream_t)stream;
    for (int r0 = 0; r0 < B; r0 += ctx->topk_rows) {
      const int Bc = (B - r0) < ctx->topk_rows ? (B - r0) : ctx->topk_rows;
      fill_common(p, ctx, H + (int64_t)r0 * ldh, ldh, W, ldw, Bc, d, V, temperature, seed, step, nullptr, 0);
      rc = run_stream_chunks(ctx, p, path, fsk::EPI_STORE, s, [&](fsk::StreamParams& c, int q0) {
        c.logits = ctx->topk_ws + (int64_t)q0 * ctx->topk_ldl;
        c.ldl = ctx->topk_ldl;
        c.tile_ratio = mask ? 0 : fsk::kXcdTileRatio;  // as the unfused call's store pass
      });
      if (rc != FS_OK) return rc;
      rc = launch_topk(ctx, ctx->topk_ws, ctx->topk_ldl, Bc, r0, V, temperature, seed, step, mask, ldm, top_k, out_idx, s);
      if (rc != FS_OK) return rc;
    }
    return FS_OK;
  }
  fill_common(p, ctx, H, ldh, W, ldw, B, d, V, temperature, seed, step, mask, ldm);
  const int nt = p.n_tiles;
  return run_stream_chunks(
      ctx, p, path, fsk::EPI_FLAT, (hipStream_t)stream,
      [&](fsk::StreamParams& c, int r0) {
        c.out_idx = out_idx + r0;
        c.dbg_max = tile_max ? tile_max + (int64_t)r0 * nt : nullptr;
        c.dbg_arg = tile_arg ? tile_arg + (int64_t)r0 * nt : nullptr;
        // tile maxima are reported over the tiling of fs_fmms_tiling; without
        // them the planner may weight the tiles per XCD (the sample does not
        // depend on the tiling)
        c.tile_ratio = tile_max ? 0 : fsk::kXcdTileRatio;
      },
      fsk::kWideMaxB, true);
}

int fs_fmms_sample_multi(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                         int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                         const uint32_t* mask, int64_t ldm, int num_samples, int32_t* out_idx, int path) {
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, V, temperature, mask, ldm, V);
  if (rc != FS_OK) return rc;
  if (!out_idx) return fail(FS_ERR_INVALID_ARG, "out_idx is NULL");
  if (num_samples < 1) return fail(FS_ERR_INVALID_ARG, "num_samples=%d must be >= 1", num_samples);
  if ((int64_t)B * num_samples > INT32_MAX)
    return fail(FS_ERR_INVALID_ARG, "B * num_samples = %lld exceeds 2^31 - 1", (long long)B * num_samples);
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  fsk::StreamParams p;
  fill_common(p, ctx, H, ldh, W, ldw, B * num_samples, d, V, temperature, seed, step, mask, ldm);
  p.samples = num_samples;
  return run_stream_chunks(
      ctx, p, path, fsk::EPI_FLAT, (hipStream_t)stream,
      [&](fsk::StreamParams& c, int r0) {
        c.out_idx = out_idx + r0;
        c.tile_ratio = fsk::kXcdTileRatio;
      },
      ctx->max_B);
}

int fs_fmms_sample_top_p(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W,
                         int64_t ldw, int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                         const uint32_t* mask, int64_t ldm, int top_k, float top_p, int32_t* out_idx, int path) {
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, V, temperature, mask, ldm, V);
  if (rc != FS_OK) return rc;
  if (!out_idx) return fail(FS_ERR_INVALID_ARG, "out_idx is NULL");
  if (top_k < 1 || top_k > ctx->max_top_k)
    return fail(top_k < 1 ? FS_ERR_INVALID_ARG : FS_ERR_CAPACITY, "top_k=%d outside [1, max_top_k=%d]", top_k,
                ctx->max_top_k);
  if (top_k > fsk::kTopkFusedMax)
    return fail(FS_ERR_UNSUPPORTED, "top-p runs on the fused top-k candidates: top_k=%d above %d", top_k,
                fsk::kTopkFusedMax);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(FS_ERR_INVALID_ARG, "top_p=%g outside (0, 1]", (double)top_p);
  if (path != FS_PATH_AUTO && path != FS_PATH_MFMA)
    return fail(path == FS_PATH_DOT ? FS_ERR_UNSUPPORTED : FS_ERR_INVALID_ARG, "path %d: top-p runs on the MFMA kernels",
                path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  return sample_topk_fused(ctx, (hipStream_t)stream, H, ldh, W, ldw, B, d, V, temperature, seed, step, mask, ldm,
                           top_k, top_p, out_idx, path);
}

int fs_unfused_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                      int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                      const uint32_t* mask, int64_t ldm, int top_k, int32_t* out_idx, float* logits_ws, int64_t ldl,
                      int path) {
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, V, temperature, mask, ldm, V);
  if (rc != FS_OK) return rc;
  if (!out_idx) return fail(FS_ERR_INVALID_ARG, "out_idx is NULL");
  if (!logits_ws || !aligned16(logits_ws)) return fail(FS_ERR_INVALID_ARG, "logits_ws must be a 16-byte aligned device pointer");
  if (ldl < V || ldl % 4 != 0) return fail(FS_ERR_INVALID_ARG, "ldl=%lld must be >= V and a multiple of 4", (long long)ldl);
  if (top_k < 0 || top_k > ctx->max_top_k)
    return fail(top_k < 0 ? FS_ERR_INVALID_ARG : FS_ERR_CAPACITY, "top_k=%d outside [0, max_top_k=%d]", top_k, ctx->max_top_k);
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipStream_t s = (hipStream_t)stream;
  fsk::StreamParams p;
  fill_common(p, ctx, H, ldh, W, ldw, B, d, V, temperature, seed, step, nullptr, 0);  // the GEMM pass ignores the mask
  rc = run_stream_chunks(ctx, p, path, fsk::EPI_STORE, s, [&](fsk::StreamParams& c, int r0) {
    c.logits = logits_ws + (int64_t)r0 * ldl;
    c.ldl = ldl;
    // the tiles of the fused call with the same mask: stored logits equal to its own bit for bit
    c.tile_ratio = mask ? 0 : fsk::kXcdTileRatio;
  });
  if (rc != FS_OK) return rc;
  if (top_k > 0) return launch_topk(ctx, logits_ws, ldl, B, 0, V, temperature, seed, step, mask, ldm, top_k, out_idx, s);
  fsk::SampleParams q;
  std::memset(&q, 0, sizeof q);
  q.logits = logits_ws;
  q.ldl = ldl;
  q.B = B;
  q.V = V;
  q.inv_t = 1.0f / temperature;
  q.seed_lo = (uint32_t)seed;
  q.seed_hi = (uint32_t)(seed >> 32);
  q.step_lo = (uint32_t)step;
  q.step_hi = (uint32_t)(step >> 32);
  q.mask = mask;
  q.ldm = ldm;
  q.n_tiles = n_tiles_for(ctx, V);
  q.ws_val = ctx->ws_val;
  q.ws_idx = ctx->ws_idx;
  q.out_idx = out_idx;
  hipError_t e = fsk::launch_sample_logits(q, s);
  if (e != hipSuccess) return hip_fail(e, "sampling kernel launch");
  return FS_OK;
}

int fs_softmax_sample(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                      int B, int d, int64_t V, float temperature, uint64_t seed, uint64_t step,
                      const uint32_t* mask, int64_t ldm, int32_t* out_idx, float* logits_ws, int64_t ldl, int path) {
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, V, temperature, mask, ldm, V);
  if (rc != FS_OK) return rc;
  if (!out_idx) return fail(FS_ERR_INVALID_ARG, "out_idx is NULL");
  if (!logits_ws || !aligned16(logits_ws)) return fail(FS_ERR_INVALID_ARG, "logits_ws must be a 16-byte aligned device pointer");
  if (ldl < V || ldl % 4 != 0) return fail(FS_ERR_INVALID_ARG, "ldl=%lld must be >= V and a multiple of 4", (long long)ldl);
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipStream_t s = (hipStream_t)stream;
  fsk::StreamParams p;
  fill_common(p, ctx, H, ldh, W, ldw, B, d, V, temperature, seed, step, nullptr, 0);
  rc = run_stream_chunks(ctx, p, path, fsk::EPI_STORE, s, [&](fsk::StreamParams& c, int r0) {
    c.logits = logits_ws + (int64_t)r0 * ldl;
    c.ldl = ldl;
    c.tile_ratio = fsk::kXcdTileRatio;  // the unmasked unfused call's tiles (this pass ignores the mask)
  });
  if (rc != FS_OK) return rc;
  fsk::CdfParams q;
  std::memset(&q, 0, sizeof q);
  q.logits = logits_ws;
  q.ldl = ldl;
  q.B = B;
  q.V = (int)V;
  q.inv_t = 1.0f / temperature;
  q.seed_lo = (uint32_t)seed;
  q.seed_hi = (uint32_t)(seed >> 32);
  q.step_lo = (uint32_t)step;
  q.step_hi = (uint32_t)(step >> 32);
  q.mask = mask;
  q.ldm = ldm;
  // about 2048 workgroups per launch, segments of at least 512 quads
  const int64_t nq = (V + 3) / 4;
  int64_t seg = 2048 / B;
  if (seg > nq / 512) seg = nq / 512;
  if (seg > fsk::kCdfMaxSeg) seg = fsk::kCdfMaxSeg;
  if (seg < 1) seg = 1;
  q.n_seg = (int)seg;
  const size_t plane = (size_t)ctx->max_B * fsk::kCdfMaxSeg;
  q.seg_m = ctx->cdf_ws;
  q.seg_z = ctx->cdf_ws + plane;
  q.seg_p = ctx->cdf_ws + 2 * plane;
  q.out_idx = out_idx;
  hipError_t e = fsk::launch_cdf_sample(q, s);
  if (e != hipSuccess) return hip_fail(e, "comparator sampling launch");
  return FS_OK;
}

int fs_group_summary(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W_group,
                     int64_t ldw, int B, int d, int64_t vocab_offset, int64_t G, float temperature, uint64_t seed,
                     uint64_t step, const uint32_t* mask, int64_t ldm, fs_group_summary_t* out, int path) {
  if (vocab_offset < 0 || vocab_offset % 32 != 0)
    return fail(FS_ERR_INVALID_ARG, "vocab_offset=%lld must be a non-negative multiple of 32", (long long)vocab_offset);
  if (G >= 1 && vocab_offset + G >= ((int64_t)1 << 31))
    return fail(FS_ERR_INVALID_ARG, "vocab_offset + G must be < 2^31");
  int rc = check_operands(ctx, H, ldh, W_group, ldw, B, d, G, temperature, mask, ldm, vocab_offset + G);
  if (rc != FS_OK) return rc;
  if (!out) return fail(FS_ERR_INVALID_ARG, "out is NULL");
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  fsk::StreamParams p;
  fill_common(p, ctx, H, ldh, W_group, ldw, B, d, G, temperature, seed, step, mask, ldm);
  p.vocab_offset = vocab_offset;
  return run_stream_chunks(ctx, p, path, fsk::EPI_GROUP, (hipStream_t)stream, [&](fsk::StreamParams& c, int r0) {
    c.out_sum = reinterpret_cast<fsk::GroupSummary*>(out + r0);
  });
}

// Summaries of n_groups consecutive groups, in launches of up to max_tiles
// groups; `ready` (may be null) makes them online: group k's tiles wait for
// ready[k] == epoch (see StreamParams::ready).
static int group_summaries(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                           int B, int d, int64_t vocab_offset, int64_t G, int n_groups, float temperature,
                           uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm, const uint32_t* ready,
                           uint32_t epoch, uint64_t wait_ticks, int32_t* status, fs_group_summary_t* out, int path) {
  if (vocab_offset < 0 || vocab_offset % 32 != 0)
    return fail(FS_ERR_INVALID_ARG, "vocab_offset=%lld must be a non-negative multiple of 32", (long long)vocab_offset);
  if (n_groups < 1) return fail(FS_ERR_INVALID_ARG, "n_groups=%d must be >= 1", n_groups);
  if (G < 16 || G % 16 != 0) return fail(FS_ERR_INVALID_ARG, "G=%lld must be a positive multiple of 16", (long long)G);
  const int64_t Vall = G * n_groups;
  if (vocab_offset + Vall >= ((int64_t)1 << 31))
    return fail(FS_ERR_INVALID_ARG, "vocab_offset + n_groups * G must be < 2^31");
  int rc = check_operands(ctx, H, ldh, W, ldw, B, d, Vall, temperature, mask, ldm, vocab_offset + Vall);
  if (rc != FS_OK) return rc;
  if (!out) return fail(FS_ERR_INVALID_ARG, "out is NULL");
  if (path < FS_PATH_AUTO || path > FS_PATH_MFMA) return fail(FS_ERR_INVALID_ARG, "unknown path %d", path);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  // launches of up to max_tiles groups, the context's tiles shared evenly
  // among them (a tile never straddles two groups)
  const int64_t gblocks = G / 16;
  for (int g0 = 0; g0 < n_groups; g0 += ctx->max_tiles) {
    const int ng = (n_groups - g0) < ctx->max_tiles ? (n_groups - g0) : ctx->max_tiles;
    int64_t tpg = ctx->max_tiles / ng;
    if (tpg > gblocks) tpg = gblocks;
    fsk::StreamParams p;
    fill_common(p, ctx, H, ldh, W + (int64_t)g0 * G * ldw, ldw, B, d, G * ng, temperature, seed, step, mask, ldm);
    p.vocab_offset = vocab_offset + (int64_t)g0 * G;
    p.group_tiles = (int)tpg;
    p.group_blocks = gblocks;
    p.n_tiles = (int)(tpg * ng);
    p.n_mblocks = gblocks * ng;
    p.group_out_stride = B;
    p.ready = ready ? ready + g0 : nullptr;
    p.ready_epoch = epoch;
    p.wait_ticks = wait_ticks;
    p.status = status;
    rc = run_stream_chunks(ctx, p, path, fsk::EPI_GROUP, (hipStream_t)stream, [&](fsk::StreamParams& c, int r0) {
      c.out_sum = reinterpret_cast<fsk::GroupSummary*>(out + (int64_t)g0 * B + r0);
    });
    if (rc != FS_OK) return rc;
  }
  return FS_OK;
}

int fs_group_summaries(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                       int B, int d, int64_t vocab_offset, int64_t G, int n_groups, float temperature, uint64_t seed,
                       uint64_t step, const uint32_t* mask, int64_t ldm, fs_group_summary_t* out, int path) {
  return group_summaries(ctx, stream, H, ldh, W, ldw, B, d, vocab_offset, G, n_groups, temperature, seed, step, mask,
                         ldm, nullptr, 0, 0, nullptr, out, path);
}

int fs_group_summaries_online(fs_ctx* ctx, void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W,
                              int64_t ldw, int B, int d, int64_t vocab_offset, int64_t G, int n_groups,
                              float temperature, uint64_t seed, uint64_t step, const uint32_t* mask, int64_t ldm,
                              const uint32_t* ready, uint32_t epoch, uint32_t max_wait_us, int32_t* status,
                              fs_group_summary_t* out, int path) {
  if (!ready || !status) return fail(FS_ERR_INVALID_ARG, "ready and status must be non-NULL");
  if (max_wait_us > 60u * 1000u * 1000u) return fail(FS_ERR_INVALID_ARG, "max_wait_us=%u exceeds 60 s", max_wait_us);
  // the wait is counted on the GPU's constant-rate real-time clock
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, ctx->device) != hipSuccess || khz <= 0)
    return fail(FS_ERR_HIP, "cannot read the wall clock rate of device %d", ctx->device);
  return group_summaries(ctx, stream, H, ldh, W, ldw, B, d, vocab_offset, G, n_groups, temperature, seed, step, mask,
                         ldm, ready, epoch, (uint64_t)max_wait_us * (uint64_t)khz / 1000u, status, out, path);
}

int fs_group_combine(fs_ctx* ctx, void* stream, const fs_group_summary_t* s, int n_groups, int B, uint64_t seed,
                     uint64_t step, int mode, int32_t* out_idx) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (!s || !out_idx) return fail(FS_ERR_INVALID_ARG, "s and out_idx must be non-NULL");
  if (n_groups < 1 || n_groups > 4096) return fail(FS_ERR_INVALID_ARG, "n_groups=%d outside [1, 4096]", n_groups);
  if (B < 1) return fail(FS_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (mode != FS_COMBINE_GUMBEL && mode != FS_COMBINE_MAX) return fail(FS_ERR_INVALID_ARG, "unknown mode %d", mode);
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipError_t e = fsk::launch_group_combine(reinterpret_cast<const fsk::GroupSummary*>(s), n_groups, B, seed, step,
                                           mode, out_idx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return FS_OK;
}

int fs_fmms_sample_noalloc(void* stream, const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw, int B,
                           int d, int64_t V, float temperature, uint64_t seed, uint64_t step, const uint32_t* mask,
                           int64_t ldm, int32_t* out_idx) {
  if (B < 1 || B > kNoAllocMaxB)
    return fail(B < 1 ? FS_ERR_INVALID_ARG : FS_ERR_CAPACITY,
                "B=%d outside [1, %d]: the allocation-free path's static scratch holds %d rows of tile winners",
                B, kNoAllocMaxB, kNoAllocMaxB);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  NoAllocDevice nd;
  const int rc = noalloc_setup(dev, nd);
  if (rc != FS_OK) return rc;
  // a context on the stack over the static scratch: the same checks, kernels and
  // tiling as fs_fmms_sample, which never allocates once given a workspace
  fs_ctx c;
  std::memset(&c, 0, sizeof c);
  c.device = dev;
  c.max_B = kNoAllocMaxB;
  c.max_V = INT32_MAX;
  c.max_top_k = 0;
  c.n_cu = nd.n_cu;
  c.max_tiles = nd.n_cu < kNoAllocMaxTiles ? nd.n_cu : kNoAllocMaxTiles;
  c.ws_val = (float*)nd.ptr;
  c.ws_idx = (int32_t*)(nd.ptr + (size_t)kNoAllocMaxB * kNoAllocMaxTiles * sizeof(float));
  return fs_fmms_sample(&c, stream, H, ldh, W, ldw, B, d, V, temperature, seed, step, mask, ldm, 0, out_idx, nullptr,
                        nullptr, FS_PATH_AUTO);
}

int fs_profile_next_launch(fs_ctx* ctx, void* before, void* after) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if ((before == nullptr) != (after == nullptr)) return fail(FS_ERR_INVALID_ARG, "before and after go together");
  ctx->prof_before = (hipEvent_t)before;
  ctx->prof_after = (hipEvent_t)after;
  return FS_OK;
}

int fs_debug_philox(fs_ctx* ctx, void* stream, uint64_t seed, uint64_t step, int row, int64_t v0, int64_t n,
                    uint32_t* r_out, float* g_out) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (n < 0 || v0 < 0 || v0 + n > ((int64_t)1 << 31) || row < 0)
    return fail(FS_ERR_INVALID_ARG, "need n >= 0, v0 >= 0, v0 + n <= 2^31, row >= 0");
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipError_t e = fsk::launch_debug_philox(seed, step, (uint32_t)row, v0, n, r_out, g_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return FS_OK;
}

int fs_debug_gumbel_bits(fs_ctx* ctx, void* stream, uint64_t r0, int64_t n, float* g_out) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (!g_out || n < 0 || r0 + (uint64_t)n > ((uint64_t)1 << 32))
    return fail(FS_ERR_INVALID_ARG, "need g_out, n >= 0 and r0 + n <= 2^32");
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipError_t e = fsk::launch_debug_gumbel_bits(r0, n, g_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return FS_OK;
}

int fs_debug_gumbel_scan(fs_ctx* ctx, void* stream, uint64_t* stats_out) {
  if (!ctx) return fail(FS_ERR_INVALID_ARG, "ctx is NULL");
  if (!stats_out) return fail(FS_ERR_INVALID_ARG, "stats_out is NULL");
  DeviceGuard guard(ctx->device);
  if (!guard.ok) return fail(FS_ERR_HIP, "cannot make device %d current", ctx->device);
  hipError_t e = fsk::launch_debug_gumbel_scan((unsigned long long*)stats_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return FS_OK;
}

}  // extern "C"
