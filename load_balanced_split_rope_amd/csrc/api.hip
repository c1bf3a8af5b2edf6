// C ABI of liblbsr: argument validation, workspace layout, kernel launches.
// The declarations and their contracts are in include/lbsr.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/lbsr.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

lbsr_status fail(lbsr_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lbsr_status fail(lbsr_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

#define LBSR_CHECK(expr)                  \
  do {                                    \
    const lbsr_status st_ = (expr);       \
    if (st_ != LBSR_OK) return st_;       \
  } while (0)

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool queried = false;
  bool gfx950 = false;
  int cu_count = 0;
  char arch[64] = {0};
};
DeviceInfo g_devices[kMaxDevices];
std::mutex g_device_mutex;

lbsr_status device_info(int device, DeviceInfo* out) {
  if (device < 0 || device >= kMaxDevices) return fail(LBSR_E_INVALID, "device %d out of range", device);
  std::lock_guard<std::mutex> lock(g_device_mutex);
  DeviceInfo& d = g_devices[device];
  if (!d.queried) {
    hipDeviceProp_t prop;
    const hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
      return fail(LBSR_E_HIP, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
    d.cu_count = prop.multiProcessorCount;
    snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.queried = true;
  }
  *out = d;
  return LBSR_OK;
}

lbsr_status current_device(DeviceInfo* out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LBSR_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  LBSR_CHECK(device_info(dev, out));
  if (!out->gfx950)
    return fail(LBSR_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, out->arch);
  return LBSR_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

lbsr_status check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(LBSR_E_INVALID, "%s is NULL", name);
  if (!aligned(p, align)) return fail(LBSR_E_INVALID, "%s is not %zu-byte aligned", name, align);
  return LBSR_OK;
}

lbsr_status check_shape(const lbsr_shape* s, int32_t batch) {
  if (!s) return fail(LBSR_E_INVALID, "shape is NULL");
  if (s->head_dim != LBSR_HEAD_DIM)
    return fail(LBSR_E_UNSUPPORTED, "head_dim %d: only 128 is supported", s->head_dim);
  if (s->page_size != LBSR_PAGE_SIZE)
    return fail(LBSR_E_UNSUPPORTED, "page_size %d: only 64 is supported", s->page_size);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(LBSR_E_INVALID, "head counts must be >= 1 (Hq %d, Hkv %d)", s->num_q_heads,
                s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(LBSR_E_INVALID, "Hq %d is not a multiple of Hkv %d", s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads / s->num_kv_heads > lbsr::kMaxGroup)
    return fail(LBSR_E_UNSUPPORTED, "group size %d > 16", s->num_q_heads / s->num_kv_heads);
  if (s->num_q_heads > 4096) return fail(LBSR_E_UNSUPPORTED, "Hq %d > 4096", s->num_q_heads);
  if (s->tokens_per_seq < 1)
    return fail(LBSR_E_INVALID, "tokens_per_seq %d < 1", s->tokens_per_seq);
  if (s->tokens_per_seq > lbsr::kMaxTokensPerSeq)
    return fail(LBSR_E_UNSUPPORTED, "tokens_per_seq %d > %d", s->tokens_per_seq,
                lbsr::kMaxTokensPerSeq);
  if (s->reserved != 0) return fail(LBSR_E_INVALID, "shape.reserved must be 0");
  if (s->kv_dtype != LBSR_KV_BF16 && s->kv_dtype != LBSR_KV_FP8_E4M3)
    return fail(LBSR_E_INVALID, "kv_dtype %d unknown", s->kv_dtype);
  if (s->max_blocks_per_seq < 1)
    return fail(LBSR_E_INVALID, "max_blocks_per_seq %d < 1", s->max_blocks_per_seq);
  if ((int64_t)s->max_blocks_per_seq * LBSR_PAGE_SIZE > INT32_MAX)
    return fail(LBSR_E_INVALID, "max_blocks_per_seq %d too large", s->max_blocks_per_seq);
  // every sequence holds its new tokens, so they fit the block table's reach
  // (kernels clamp lengths up to the token count and walk that many rows)
  if ((int64_t)s->tokens_per_seq > (int64_t)s->max_blocks_per_seq * LBSR_PAGE_SIZE)
    return fail(LBSR_E_INVALID, "tokens_per_seq %d > max_blocks_per_seq %d x %d rows",
                s->tokens_per_seq, s->max_blocks_per_seq, LBSR_PAGE_SIZE);
  if (s->num_pages < 1 || s->num_pages > INT32_MAX)
    return fail(LBSR_E_INVALID, "num_pages %lld out of [1, 2^31)", (long long)s->num_pages);
  if (s->page_stride < LBSR_TILE_ELEMS || s->page_stride % LBSR_TILE_ELEMS ||
      s->head_stride < LBSR_TILE_ELEMS || s->head_stride % LBSR_TILE_ELEMS)
    return fail(LBSR_E_INVALID, "page_stride %lld / head_stride %lld must be positive multiples of 8192",
                (long long)s->page_stride, (long long)s->head_stride);
  // offsets page * page_stride + head * head_stride stay far inside int64:
  // each term (and so a pool's extent) is bounded by 2^46 elements, more than
  // any device holds
  constexpr int64_t kMaxPoolElems = (int64_t)1 << 46;
  if (s->page_stride > kMaxPoolElems / s->num_pages ||
      s->head_stride > kMaxPoolElems / s->num_kv_heads)
    return fail(LBSR_E_INVALID, "page_stride %lld / head_stride %lld: a pool would exceed 2^46 elements",
                (long long)s->page_stride, (long long)s->head_stride);
  const bool page_major = s->page_stride >= (int64_t)s->num_kv_heads * s->head_stride;
  const bool head_major = s->head_stride >= s->num_pages * s->page_stride;
  if (!page_major && !head_major)
    return fail(LBSR_E_INVALID, "page_stride/head_stride make tiles overlap");
  if (batch < 1) return fail(LBSR_E_INVALID, "batch %d < 1", batch);
  // the prologue runs at most one wave per (new token, row): the count must fit an int
  if ((int64_t)batch * s->tokens_per_seq * (s->num_q_heads + 2 * s->num_kv_heads) > INT32_MAX / 2)
    return fail(LBSR_E_UNSUPPORTED, "batch %d x tokens_per_seq %d is too many rows", batch,
                s->tokens_per_seq);
  if (batch > lbsr::kMaxBatch)
    return fail(LBSR_E_UNSUPPORTED, "batch %d > %d", batch, lbsr::kMaxBatch);
  if ((int64_t)batch * s->max_blocks_per_seq > INT32_MAX)
    return fail(LBSR_E_UNSUPPORTED, "batch * max_blocks_per_seq exceeds 2^31 tiles");
  return LBSR_OK;
}

lbsr_status check_params(const lbsr_params* p, int32_t kv_dtype) {
  if (!p) return fail(LBSR_E_INVALID, "params is NULL");
  if (!(p->rope_theta > 0) || !isfinite(p->rope_theta))
    return fail(LBSR_E_INVALID, "rope_theta %g must be finite and > 0", p->rope_theta);
  if (!(p->rms_eps >= 0) || !isfinite(p->rms_eps))
    return fail(LBSR_E_INVALID, "rms_eps %g must be finite and >= 0", (double)p->rms_eps);
  if (p->norm_before_rope != 0 && p->norm_before_rope != 1)
    return fail(LBSR_E_INVALID, "norm_before_rope must be 0 or 1");
  if (!(p->sm_scale >= 0) || !isfinite(p->sm_scale))
    return fail(LBSR_E_INVALID, "sm_scale %g must be finite and >= 0", (double)p->sm_scale);
  if (p->out_dtype != LBSR_OUT_BF16 && p->out_dtype != LBSR_OUT_FP8_E4M3)
    return fail(LBSR_E_INVALID, "out_dtype %d unknown", p->out_dtype);
  if (p->out_dtype == LBSR_OUT_FP8_E4M3 && (!(p->out_scale > 0) || !isfinite(p->out_scale)))
    return fail(LBSR_E_INVALID, "out_scale %g must be finite and > 0", (double)p->out_scale);
  if (kv_dtype == LBSR_KV_FP8_E4M3 &&
      (!(p->k_scale > 0) || !isfinite(p->k_scale) || !(p->v_scale > 0) || !isfinite(p->v_scale)))
    return fail(LBSR_E_INVALID, "k_scale %g / v_scale %g must be finite and > 0",
                (double)p->k_scale, (double)p->v_scale);
  if (p->qk_dtype != LBSR_QK_BF16 && p->qk_dtype != LBSR_QK_FP8_E4M3)
    return fail(LBSR_E_INVALID, "qk_dtype %d unknown", p->qk_dtype);
  if (p->qk_dtype == LBSR_QK_FP8_E4M3) {
    if (kv_dtype != LBSR_KV_FP8_E4M3)
      return fail(LBSR_E_UNSUPPORTED, "qk_dtype FP8 needs an FP8 cache");
    if (!(p->q_scale > 0) || !isfinite(p->q_scale) || !isfinite(1.0f / p->q_scale))
      return fail(LBSR_E_INVALID, "q_scale %g must be finite and > 0 with a finite inverse",
                  (double)p->q_scale);
  }
  return LBSR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The decode attention path (split + merge) holds one KV head's (new token,
// q head) columns in at most 4 matrix-core column blocks.
lbsr_status check_columns(const lbsr_shape* s) {
  if ((int64_t)s->tokens_per_seq * (s->num_q_heads / s->num_kv_heads) > lbsr::kMaxColumns)
    return fail(LBSR_E_UNSUPPORTED, "tokens_per_seq %d x group %d > %d (use the prefill path)",
                s->tokens_per_seq, s->num_q_heads / s->num_kv_heads, lbsr::kMaxColumns);
  return LBSR_OK;
}

lbsr_status compute_layout(const lbsr_shape* shape, int32_t batch, const lbsr_sched_cfg* cfg,
                           lbsr_ws_layout* out) {
  LBSR_CHECK(check_shape(shape, batch));
  LBSR_CHECK(check_columns(shape));
  if (!cfg) return fail(LBSR_E_INVALID, "cfg is NULL");
  if (!out) return fail(LBSR_E_INVALID, "out is NULL");
  if (cfg->sched != LBSR_SCHED_DYNAMIC && cfg->sched != LBSR_SCHED_STATIC)
    return fail(LBSR_E_INVALID, "sched %d unknown", cfg->sched);
  if (cfg->flags & ~LBSR_SCHED_FOLD_MERGE)
    return fail(LBSR_E_INVALID, "cfg.flags 0x%x has unknown bits", (unsigned)cfg->flags);
  if (cfg->flags & LBSR_SCHED_FOLD_MERGE) {
    const int G = shape->num_q_heads / shape->num_kv_heads;
    if (shape->tokens_per_seq != 1)
      return fail(LBSR_E_UNSUPPORTED, "LBSR_SCHED_FOLD_MERGE needs tokens_per_seq = 1, not %d",
                  shape->tokens_per_seq);
    if (G & (G - 1))
      return fail(LBSR_E_UNSUPPORTED, "LBSR_SCHED_FOLD_MERGE needs a power-of-two group, not %d", G);
  }
  // a sequence gets at most one chunk per worker or split; the merge handles 1024
  if (cfg->num_workers < 0 || cfg->num_workers > 1024)
    return fail(LBSR_E_INVALID, "num_workers %d out of [0, 1024]", cfg->num_workers);
  if (cfg->static_splits < 0 || cfg->static_splits > 1024)
    return fail(LBSR_E_INVALID, "static_splits %d out of [0, 1024]", cfg->static_splits);
  int nonzero = 0;
  for (int x = 0; x < LBSR_NUM_XCDS; ++x) {
    const int32_t wt = cfg->xcd_weight[x];
    if (wt < 0 || wt > LBSR_MAX_XCD_WEIGHT)
      return fail(LBSR_E_INVALID, "xcd_weight[%d] = %d out of [0, %d]", x, wt, LBSR_MAX_XCD_WEIGHT);
    nonzero += wt != 0;
  }
  if (nonzero != 0 && nonzero != LBSR_NUM_XCDS)
    return fail(LBSR_E_INVALID, "xcd_weight must be all 0 or all in [1, %d]", LBSR_MAX_XCD_WEIGHT);
  if (nonzero != 0 && cfg->sched != LBSR_SCHED_DYNAMIC)
    return fail(LBSR_E_INVALID, "xcd_weight applies to the dynamic schedule only");
  int32_t P = cfg->num_workers;
  if (P == 0) {
    DeviceInfo d;
    LBSR_CHECK(current_device(&d));
    P = d.cu_count;
  }
  int64_t W, cmax;
  int32_t S = 0;
  if (cfg->sched == LBSR_SCHED_DYNAMIC) {
    W = P;
    cmax = (int64_t)P + batch - 1;
  } else {
    S = cfg->static_splits ? cfg->static_splits : (P / batch > 1 ? P / batch : 1);
    W = (int64_t)batch * S;
    cmax = W;
  }
  if (W > (1 << 22)) return fail(LBSR_E_UNSUPPORTED, "%lld workers is too many", (long long)W);
  {
    // the merge stages (chunks of one sequence) x (columns of a KV head) weights in LDS
    const int64_t per_seq = cfg->sched == LBSR_SCHED_DYNAMIC ? P : S;
    const int64_t rows = per_seq < shape->max_blocks_per_seq ? per_seq : shape->max_blocks_per_seq;
    const int64_t cols = (int64_t)shape->tokens_per_seq * (shape->num_q_heads / shape->num_kv_heads);
    if (rows * cols * 4 > lbsr::kMergeLdsBytes)
      return fail(LBSR_E_UNSUPPORTED,
                  "%lld chunks per sequence x %lld columns exceed the merge's %d-byte LDS stage",
                  (long long)rows, (long long)cols, lbsr::kMergeLdsBytes);
  }
  const int64_t Hq = shape->num_q_heads;
  const int64_t Tq = shape->tokens_per_seq;
  size_t off = 0;
  memset(out, 0, sizeof *out);
  out->error_word = off;   off = align256(off + 4);
  out->cu_tiles = off;     off = align256(off + 4 * (size_t)(batch + 1));
  out->worker_chunk = off; off = align256(off + 4 * (size_t)(W + 1));
  out->chunks = off;       off = align256(off + 16 * (size_t)cmax);
  out->seq_chunk = off;    off = align256(off + 4 * (size_t)(batch + 1));
  out->seq_len_eff = off;  off = align256(off + 4 * (size_t)batch);
  out->token_status = off; off = align256(off + 4 * (size_t)batch * Tq);
  out->partial_o = off;    off = align256(off + 4 * (size_t)cmax * Tq * Hq * LBSR_HEAD_DIM);
  out->partial_lse = off;  off = align256(off + 4 * (size_t)cmax * Tq * Hq);
  out->arrivals = off;     off = align256(off + 4 * (size_t)batch * shape->num_kv_heads);
  out->total = off;
  out->num_workers = (int32_t)W;
  out->max_chunks = (int32_t)cmax;
  out->static_splits = S;
  return LBSR_OK;
}

lbsr::PlanPtrs plan_ptrs(void* ws, const lbsr_ws_layout& l) {
  char* base = (char*)ws;
  lbsr::PlanPtrs p;
  p.error_word = (int32_t*)(base + l.error_word);
  p.cu_tiles = (int32_t*)(base + l.cu_tiles);
  p.worker_chunk = (int32_t*)(base + l.worker_chunk);
  p.chunks = (int32_t*)(base + l.chunks);
  p.seq_chunk = (int32_t*)(base + l.seq_chunk);
  p.seq_len_eff = (int32_t*)(base + l.seq_len_eff);
  p.token_status = (int32_t*)(base + l.token_status);
  p.partial_o = (float*)(base + l.partial_o);
  p.partial_lse = (float*)(base + l.partial_lse);
  p.arrivals = (int32_t*)(base + l.arrivals);
  return p;
}

lbsr::Geometry geometry(const lbsr_shape* s, int32_t batch) {
  lbsr::Geometry g;
  g.batch = batch;
  g.num_q_heads = s->num_q_heads;
  g.num_kv_heads = s->num_kv_heads;
  g.group = s->num_q_heads / s->num_kv_heads;
  g.max_blocks = s->max_blocks_per_seq;
  g.tokens = s->tokens_per_seq;
  g.num_pages = s->num_pages;
  g.page_stride = s->page_stride;
  g.head_stride = s->head_stride;
  return g;
}

lbsr_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LBSR_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return LBSR_OK;
}

lbsr_status check_workspace(void* ws, size_t ws_bytes, const lbsr_ws_layout& l) {
  LBSR_CHECK(check_ptr(ws, 256, "workspace"));
  if (ws_bytes < l.total)
    return fail(LBSR_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, l.total);
  return LBSR_OK;
}

// ---- the four stages, validated separately so each entry point can reuse them ----

lbsr_status validate_prologue(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                              const void* q, const void* k, const void* v, const int32_t* positions,
                              const void* wq, const void* wk, const int32_t* bt, void* kc, void* vc,
                              void* q_out, const int32_t* error_word) {
  LBSR_CHECK(check_shape(shape, batch));
  LBSR_CHECK(check_params(params, shape->kv_dtype));
  LBSR_CHECK(check_ptr(q, 16, "q"));
  LBSR_CHECK(check_ptr(k, 16, "k"));
  LBSR_CHECK(check_ptr(v, 16, "v"));
  LBSR_CHECK(check_ptr(positions, 4, "positions"));
  LBSR_CHECK(check_ptr(wq, 16, "q_norm_w"));
  LBSR_CHECK(check_ptr(wk, 16, "k_norm_w"));
  LBSR_CHECK(check_ptr(bt, 4, "block_table"));
  LBSR_CHECK(check_ptr(kc, 16, "k_cache"));
  LBSR_CHECK(check_ptr(vc, 16, "v_cache"));
  LBSR_CHECK(check_ptr(q_out, 16, "q_out"));
  if (error_word && !aligned(error_word, 4)) return fail(LBSR_E_INVALID, "error_word misaligned");
  if (q_out == q) return fail(LBSR_E_INVALID, "q_out may not alias q");
  return LBSR_OK;
}

lbsr_status validate_attention(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                               const void* q_out, const void* kc, const void* vc, const int32_t* bt,
                               void* out, const float* lse_out) {
  LBSR_CHECK(check_shape(shape, batch));
  LBSR_CHECK(check_params(params, shape->kv_dtype));
  LBSR_CHECK(check_ptr(q_out, 16, "q_out"));
  LBSR_CHECK(check_ptr(kc, 16, "k_cache"));
  LBSR_CHECK(check_ptr(vc, 16, "v_cache"));
  LBSR_CHECK(check_ptr(bt, 4, "block_table"));
  LBSR_CHECK(check_ptr(out, 16, "out"));
  if (lse_out && !aligned(lse_out, 4)) return fail(LBSR_E_INVALID, "lse_out misaligned");
  return LBSR_OK;
}

// theta^(-2i/128) for i < 64, with the host's libm; the last theta's table is
// kept per thread, as a step normally reuses it.
const lbsr::RopeFreqs& rope_freqs(double theta) {
  thread_local double cached_theta = 0.0;
  thread_local lbsr::RopeFreqs table;
  if (theta != cached_theta) {
    for (int i = 0; i < LBSR_HEAD_DIM / 2; ++i)
      table.omega[i] = pow(theta, (-2.0 * (double)i) / (double)LBSR_HEAD_DIM);
    cached_theta = theta;
  }
  return table;
}

lbsr_status run_prologue(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                         const void* q, const void* k, const void* v, const int32_t* positions,
                         const void* wq, const void* wk, const int32_t* bt, void* kc, void* vc,
                         void* q_out, int32_t* error_word, hipStream_t stream,
                         int32_t total_tokens = -1, const int32_t* q_start = nullptr) {
  const lbsr::Geometry geo = geometry(shape, batch);
  const bool fp8 = shape->kv_dtype == LBSR_KV_FP8_E4M3;
  const int num_tokens = q_start ? total_tokens : batch * shape->tokens_per_seq;
  return hip_status(lbsr::launch_prologue(geo, fp8, q, k, v, positions, wq, wk, bt, kc, vc, q_out,
                                          error_word, rope_freqs(params->rope_theta),
                                          (double)params->rms_eps,
                                          params->norm_before_rope, fp8 ? params->k_scale : 1.0,
                                          fp8 ? params->v_scale : 1.0, num_tokens, q_start,
                                          stream),
                    "prologue launch");
}

bool folded(const lbsr_sched_cfg* cfg) { return (cfg->flags & LBSR_SCHED_FOLD_MERGE) != 0; }

lbsr::SchedParams sched_params(const lbsr_shape* shape, const lbsr_sched_cfg* cfg,
                               const lbsr_ws_layout& l) {
  lbsr::SchedParams sp{};
  sp.min_len = shape->tokens_per_seq;
  sp.dynamic = cfg->sched == LBSR_SCHED_DYNAMIC;
  sp.num_workers = l.num_workers;
  sp.splits = l.static_splits;
  sp.weighted = sp.dynamic && cfg->xcd_weight[0] != 0;  // validated: all zero or all positive
  for (int x = 0; x < lbsr::kXcds; ++x) sp.xcd_weight[x] = sp.weighted ? cfg->xcd_weight[x] : 1;
  sp.fold_groups = folded(cfg) ? shape->num_kv_heads : 0;
  return sp;
}

lbsr_status run_plan(const lbsr_shape* shape, int32_t batch, const int32_t* seq_lens,
                     const lbsr_sched_cfg* cfg, const lbsr_ws_layout& l, void* ws, hipStream_t stream) {
  return hip_status(lbsr::launch_plan(seq_lens, batch, shape->max_blocks_per_seq,
                                      sched_params(shape, cfg, l), plan_ptrs(ws, l), stream),
                    "plan launch");
}

lbsr_status run_plan_prologue(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                              const int32_t* seq_lens, const lbsr_sched_cfg* cfg,
                              const lbsr_ws_layout& l, void* ws, const void* q, const void* k,
                              const void* v, const int32_t* positions, const void* wq,
                              const void* wk, const int32_t* bt, void* kc, void* vc, void* q_out,
                              hipStream_t stream) {
  const lbsr::Geometry geo = geometry(shape, batch);
  const bool fp8 = shape->kv_dtype == LBSR_KV_FP8_E4M3;
  return hip_status(
      lbsr::launch_plan_prologue(seq_lens, sched_params(shape, cfg, l), plan_ptrs(ws, l), geo, fp8, q,
                                 k, v, positions,
                                 wq, wk, bt, kc, vc, q_out, rope_freqs(params->rope_theta),
                                 (double)params->rms_eps, params->norm_before_rope,
                                 fp8 ? params->k_scale : 1.0, fp8 ? params->v_scale : 1.0, stream),
      "plan + prologue launch");
}

bool qk_fp8(const lbsr_params* p) { return p->qk_dtype == LBSR_QK_FP8_E4M3; }

// 1/q_scale rounded to fp32: q codes are RNE(q * this), the product in fp32.
float inv_q_scale(const lbsr_params* p) { return qk_fp8(p) ? 1.0f / p->q_scale : 1.0f; }

float score_scale_log2(const lbsr_params* p, int32_t kv_dtype) {
  const double sm = p->sm_scale > 0 ? (double)p->sm_scale : 1.0 / sqrt((double)LBSR_HEAD_DIM);
  const double ks = kv_dtype == LBSR_KV_FP8_E4M3 ? (double)p->k_scale : 1.0;
  const double qs = qk_fp8(p) ? (double)p->q_scale : 1.0;   // FP8 scores are of q's codes
  return (float)(sm * ks * qs * 1.4426950408889634074);
}

lbsr_status run_split(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                      const void* q_out, const void* kc, const void* vc, const int32_t* bt,
                      const lbsr_ws_layout& l, void* ws, void* out, float* lse_out,
                      int64_t* trace, bool fold, bool fold_status, hipStream_t stream) {
  const lbsr::Geometry geo = geometry(shape, batch);
  const bool fp8 = shape->kv_dtype == LBSR_KV_FP8_E4M3;
  // outputs and partials carry o / out_scale (FP8 output), V's scale folded in
  const bool out_fp8 = params->out_dtype == LBSR_OUT_FP8_E4M3;
  const double vs = fp8 ? (double)params->v_scale : 1.0;
  const float o_scale = (float)(out_fp8 ? vs / (double)params->out_scale : vs);
  return hip_status(lbsr::launch_split_attention(geo, fp8, out_fp8, qk_fp8(params), fold,
                                                 fold_status, l.num_workers, q_out, kc, vc, bt,
                                                 plan_ptrs(ws, l), out, lse_out,
                                                 score_scale_log2(params, shape->kv_dtype),
                                                 o_scale, inv_q_scale(params), trace, stream),
                    "split attention launch");
}

lbsr_status run_combine(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                        const lbsr_ws_layout& l, void* ws, void* out, float* lse_out,
                        bool fold_token_status, hipStream_t stream) {
  const lbsr::Geometry geo = geometry(shape, batch);
  // a sequence has at most one chunk per worker (dynamic) or split (static),
  // and at most one per tile: the merge stages that many rows' lse in LDS
  const int per_seq = l.static_splits ? l.static_splits : l.num_workers;
  const int bound = per_seq < shape->max_blocks_per_seq ? per_seq : shape->max_blocks_per_seq;
  return hip_status(lbsr::launch_combine(geo, plan_ptrs(ws, l), out, lse_out, bound,
                                         params->out_dtype == LBSR_OUT_FP8_E4M3,
                                         fold_token_status, stream),
                    "merge launch");
}

lbsr_status run_prefill(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                        const void* q_out, const void* kc, const void* vc, const int32_t* bt,
                        const int32_t* seq_lens, void* out, float* lse_out, int32_t* error_word,
                        hipStream_t stream, int32_t total_tokens = -1,
                        const int32_t* q_start = nullptr, void* work = nullptr) {
  const lbsr::Geometry geo = geometry(shape, batch);
  const bool fp8 = shape->kv_dtype == LBSR_KV_FP8_E4M3;
  const bool out_fp8 = params->out_dtype == LBSR_OUT_FP8_E4M3;
  const double vs = fp8 ? (double)params->v_scale : 1.0;
  const float o_scale = (float)(out_fp8 ? vs / (double)params->out_scale : vs);
  return hip_status(lbsr::launch_prefill(geo, fp8, out_fp8, q_out, kc, vc, bt, seq_lens, out,
                                         lse_out, score_scale_log2(params, shape->kv_dtype),
                                         o_scale, error_word, q_start, total_tokens,
                                         (int32_t*)work, qk_fp8(params), inv_q_scale(params),
                                         stream),
                    "prefill launch");
}

lbsr_status validate_prefill(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                             const void* q_out, const void* kc, const void* vc, const int32_t* bt,
                             const int32_t* seq_lens, void* out, const float* lse_out,
                             const int32_t* error_word) {
  LBSR_CHECK(check_shape(shape, batch));
  LBSR_CHECK(check_params(params, shape->kv_dtype));
  LBSR_CHECK(check_ptr(q_out, 16, "q_out"));
  LBSR_CHECK(check_ptr(kc, 16, "k_cache"));
  LBSR_CHECK(check_ptr(vc, 16, "v_cache"));
  LBSR_CHECK(check_ptr(bt, 4, "block_table"));
  LBSR_CHECK(check_ptr(seq_lens, 4, "seq_lens"));
  LBSR_CHECK(check_ptr(out, 16, "out"));
  if (lse_out && !aligned(lse_out, 4)) return fail(LBSR_E_INVALID, "lse_out misaligned");
  if (error_word && !aligned(error_word, 4)) return fail(LBSR_E_INVALID, "error_word misaligned");
  // one workgroup per (block of new tokens, sequence, KV head)
  const int64_t per = lbsr::kPrefillColumns / (shape->num_q_heads / shape->num_kv_heads);
  const int64_t grid = (shape->tokens_per_seq + per - 1) / per * batch * shape->num_kv_heads;
  if (grid > INT32_MAX) return fail(LBSR_E_UNSUPPORTED, "prefill grid of %lld workgroups", (long long)grid);
  return LBSR_OK;
}

// Bytes of a prefill's workspace: header + one int2 per work item.
size_t prefill_workspace_bytes(const lbsr_shape* shape, int32_t batch, int32_t total_tokens) {
  const int64_t tpb = lbsr::kPrefillColumns / (shape->num_q_heads / shape->num_kv_heads);
  const int64_t items = (total_tokens + tpb - 1) / tpb + batch;
  return (size_t)lbsr::kPrefillListOffset + 8 * (size_t)items;
}

// The ragged batch's extra arguments: the packed token count, q_start and the
// workspace of the work list.
lbsr_status validate_varlen(const lbsr_shape* shape, int32_t batch, int32_t total_tokens,
                            const int32_t* q_start, void* ws, size_t ws_bytes) {
  if (total_tokens < 0) return fail(LBSR_E_INVALID, "total_tokens %d < 0", total_tokens);
  const int64_t rows = shape->num_q_heads + 2 * shape->num_kv_heads;
  if ((int64_t)total_tokens * rows > INT32_MAX / 2)
    return fail(LBSR_E_UNSUPPORTED, "total_tokens %d is too many rows", total_tokens);
  LBSR_CHECK(check_ptr(q_start, 4, "q_start"));
  LBSR_CHECK(check_ptr(ws, 256, "workspace"));
  const size_t need = prefill_workspace_bytes(shape, batch, total_tokens);
  if (ws_bytes < need)
    return fail(LBSR_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return LBSR_OK;
}

// The uniform prefill's optional workspace (the sorted work list): null, or
// large enough for batch * tokens_per_seq tokens.
lbsr_status validate_uniform_workspace(const lbsr_shape* shape, int32_t batch, void* ws,
                                       size_t ws_bytes) {
  if (!ws) return LBSR_OK;
  LBSR_CHECK(check_ptr(ws, 256, "workspace"));
  const size_t need = prefill_workspace_bytes(shape, batch, batch * shape->tokens_per_seq);
  if (ws_bytes < need)
    return fail(LBSR_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return LBSR_OK;
}

}  // namespace

// ---- scratch for the step that allocates nothing (lbsr_decode_step_noalloc) ----
// One file-scope device array per GPU holds that call's workspace.  In host
// code `scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[LBSR_NOALLOC_SCRATCH_BYTES];

namespace {

void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

lbsr_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LBSR_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LBSR_E_INVALID, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LBSR_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LBSR_OK;
}

}  // namespace

extern "C" {

int32_t lbsr_abi_version(void) { return LBSR_ABI_VERSION; }

const char* lbsr_status_string(lbsr_status status) {
  switch (status) {
    case LBSR_OK: return "LBSR_OK";
    case LBSR_E_INVALID: return "LBSR_E_INVALID: invalid argument";
    case LBSR_E_UNSUPPORTED: return "LBSR_E_UNSUPPORTED: unsupported shape or device";
    case LBSR_E_WORKSPACE: return "LBSR_E_WORKSPACE: workspace too small";
    case LBSR_E_HIP: return "LBSR_E_HIP: HIP runtime error";
  }
  return "unknown lbsr_status";
}

const char* lbsr_last_error(void) { return g_last_error; }

lbsr_status lbsr_device_workers(int device, int32_t* out) {
  g_last_error[0] = 0;
  if (!out) return fail(LBSR_E_INVALID, "out is NULL");
  DeviceInfo d;
  LBSR_CHECK(device_info(device, &d));
  if (!d.gfx950)
    return fail(LBSR_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950", device, d.arch);
  *out = d.cu_count;
  return LBSR_OK;
}

lbsr_status lbsr_workspace_layout(const lbsr_shape* shape, int32_t batch, const lbsr_sched_cfg* cfg,
                                  lbsr_ws_layout* out) {
  g_last_error[0] = 0;
  return compute_layout(shape, batch, cfg, out);
}

lbsr_status lbsr_workspace_size(const lbsr_shape* shape, int32_t batch, const lbsr_sched_cfg* cfg,
                                size_t* bytes) {
  g_last_error[0] = 0;
  if (!bytes) return fail(LBSR_E_INVALID, "bytes is NULL");
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  *bytes = l.total;
  return LBSR_OK;
}

lbsr_status lbsr_rope_norm_kv_write(const lbsr_shape* shape, const lbsr_params* params,
                                    int32_t batch, const void* q, const void* k, const void* v,
                                    const int32_t* positions, const void* q_norm_w,
                                    const void* k_norm_w, const int32_t* block_table,
                                    void* k_cache, void* v_cache, void* q_out, int32_t* error_word,
                                    void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                               block_table, k_cache, v_cache, q_out, error_word));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  return run_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w, block_table,
                      k_cache, v_cache, q_out, error_word, (hipStream_t)stream);
}

lbsr_status lbsr_plan(const lbsr_shape* shape, int32_t batch, const int32_t* seq_lens,
                      const lbsr_sched_cfg* cfg, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  LBSR_CHECK(check_ptr(seq_lens, 4, "seq_lens"));
  LBSR_CHECK(check_workspace(workspace, ws_bytes, l));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  return run_plan(shape, batch, seq_lens, cfg, l, workspace, (hipStream_t)stream);
}

lbsr_status lbsr_attention(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                           const void* q_out, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const lbsr_sched_cfg* cfg, void* workspace,
                           size_t ws_bytes, void* out, float* lse_out, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_attention(shape, params, batch, q_out, k_cache, v_cache, block_table, out,
                                lse_out));
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  LBSR_CHECK(check_workspace(workspace, ws_bytes, l));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  const hipStream_t s = (hipStream_t)stream;
  LBSR_CHECK(run_split(shape, params, batch, q_out, k_cache, v_cache, block_table, l, workspace, out,
                       lse_out, nullptr, folded(cfg), false, s));
  if (folded(cfg)) return LBSR_OK;   // merged inside the split launch
  return run_combine(shape, params, batch, l, workspace, out, lse_out, false, s);
}

static lbsr_status decode_step_impl(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                                    const void* q, const void* k, const void* v,
                                    const int32_t* positions, const int32_t* seq_lens,
                                    const void* q_norm_w, const void* k_norm_w,
                                    const int32_t* block_table, void* k_cache, void* v_cache,
                                    void* q_out, const lbsr_sched_cfg* cfg, void* workspace,
                                    size_t ws_bytes, void* out, float* lse_out, void* stream,
                                    float* kernel_ms, int64_t* trace) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                               block_table, k_cache, v_cache, q_out, nullptr));
  LBSR_CHECK(validate_attention(shape, params, batch, q_out, k_cache, v_cache, block_table, out,
                                lse_out));
  LBSR_CHECK(check_ptr(seq_lens, 4, "seq_lens"));
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  LBSR_CHECK(check_workspace(workspace, ws_bytes, l));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  const hipStream_t s = (hipStream_t)stream;

  hipEvent_t ev[4] = {};
  if (kernel_ms) {
    for (int i = 0; i < 4; ++i) {
      const hipError_t e = hipEventCreate(&ev[i]);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
        return hip_status(e, "hipEventCreate");
      }
    }
  }
  lbsr_status st = LBSR_OK;
  auto mark = [&](int i) {
    if (kernel_ms && st == LBSR_OK) st = hip_status(hipEventRecord(ev[i], s), "hipEventRecord");
  };
  // One launch computes the schedule and the prologue; they are independent.
  mark(0);
  if (st == LBSR_OK)
    st = run_plan_prologue(shape, params, batch, seq_lens, cfg, l, workspace, q, k, v, positions,
                           q_norm_w, k_norm_w, block_table, k_cache, v_cache, q_out, s);
  mark(1);
  if (st == LBSR_OK)
    st = run_split(shape, params, batch, q_out, k_cache, v_cache, block_table, l, workspace, out,
                   lse_out, trace, folded(cfg), true, s);
  mark(2);
  // folded: merged inside the split launch (its time then shows as 0 here)
  if (st == LBSR_OK && !folded(cfg))
    st = run_combine(shape, params, batch, l, workspace, out, lse_out, true, s);
  mark(3);
  if (kernel_ms) {
    if (st == LBSR_OK) st = hip_status(hipEventSynchronize(ev[3]), "hipEventSynchronize");
    for (int i = 0; i < 3 && st == LBSR_OK; ++i)
      st = hip_status(hipEventElapsedTime(&kernel_ms[i], ev[i], ev[i + 1]), "hipEventElapsedTime");
    for (int i = 0; i < 4; ++i) (void)hipEventDestroy(ev[i]);
  }
  return st;
}

lbsr_status lbsr_prefill_attention(const lbsr_shape* shape, const lbsr_params* params,
                                   int32_t batch, const void* q_out, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, void* workspace, size_t ws_bytes,
                                   void* out, float* lse_out, int32_t* error_word, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table,
                              seq_lens, out, lse_out, error_word));
  LBSR_CHECK(validate_uniform_workspace(shape, batch, workspace, ws_bytes));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  return run_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table, seq_lens, out,
                     lse_out, error_word, (hipStream_t)stream, batch * shape->tokens_per_seq,
                     nullptr, workspace);
}

lbsr_status lbsr_prefill_step(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                              const void* q, const void* k, const void* v,
                              const int32_t* positions, const int32_t* seq_lens,
                              const void* q_norm_w, const void* k_norm_w,
                              const int32_t* block_table, void* k_cache, void* v_cache,
                              void* q_out, void* workspace, size_t ws_bytes, void* out,
                              float* lse_out, int32_t* error_word, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                               block_table, k_cache, v_cache, q_out, error_word));
  LBSR_CHECK(validate_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table,
                              seq_lens, out, lse_out, error_word));
  LBSR_CHECK(validate_uniform_workspace(shape, batch, workspace, ws_bytes));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  const hipStream_t s = (hipStream_t)stream;
  LBSR_CHECK(run_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                          block_table, k_cache, v_cache, q_out, error_word, s));
  return run_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table, seq_lens, out,
                     lse_out, error_word, s, batch * shape->tokens_per_seq, nullptr, workspace);
}

lbsr_status lbsr_prefill_attention_varlen(const lbsr_shape* shape, const lbsr_params* params,
                                          int32_t batch, int32_t total_tokens,
                                          const int32_t* q_start, const void* q_out,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          void* workspace, size_t ws_bytes, void* out,
                                          float* lse_out, int32_t* error_word, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table,
                              seq_lens, out, lse_out, error_word));
  LBSR_CHECK(validate_varlen(shape, batch, total_tokens, q_start, workspace, ws_bytes));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  if (total_tokens == 0) return LBSR_OK;
  return run_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table, seq_lens, out,
                     lse_out, error_word, (hipStream_t)stream, total_tokens, q_start,
                     workspace);
}

lbsr_status lbsr_prefill_workspace_size(const lbsr_shape* shape, int32_t batch,
                                        int32_t total_tokens, size_t* bytes) {
  g_last_error[0] = 0;
  if (!bytes) return fail(LBSR_E_INVALID, "bytes is null");
  LBSR_CHECK(check_shape(shape, batch));
  if (total_tokens < 0) return fail(LBSR_E_INVALID, "total_tokens %d < 0", total_tokens);
  *bytes = prefill_workspace_bytes(shape, batch, total_tokens);
  return LBSR_OK;
}

lbsr_status lbsr_prefill_step_varlen(const lbsr_shape* shape, const lbsr_params* params,
                                     int32_t batch, int32_t total_tokens,
                                     const int32_t* q_start, const void* q, const void* k,
                                     const void* v, const int32_t* positions,
                                     const int32_t* seq_lens, const void* q_norm_w,
                                     const void* k_norm_w, const int32_t* block_table,
                                     void* k_cache, void* v_cache, void* q_out,
                                     void* workspace, size_t ws_bytes, void* out,
                                     float* lse_out, int32_t* error_word, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(validate_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                               block_table, k_cache, v_cache, q_out, error_word));
  LBSR_CHECK(validate_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table,
                              seq_lens, out, lse_out, error_word));
  LBSR_CHECK(validate_varlen(shape, batch, total_tokens, q_start, workspace, ws_bytes));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  if (total_tokens == 0) return LBSR_OK;
  const hipStream_t s = (hipStream_t)stream;
  LBSR_CHECK(run_prologue(shape, params, batch, q, k, v, positions, q_norm_w, k_norm_w,
                          block_table, k_cache, v_cache, q_out, error_word, s, total_tokens,
                          q_start));
  return run_prefill(shape, params, batch, q_out, k_cache, v_cache, block_table, seq_lens, out,
                     lse_out, error_word, s, total_tokens, q_start, workspace);
}

lbsr_status lbsr_decode_step(const lbsr_shape* shape, const lbsr_params* params, int32_t batch,
                             const void* q, const void* k, const void* v, const int32_t* positions,
                             const int32_t* seq_lens, const void* q_norm_w, const void* k_norm_w,
                             const int32_t* block_table, void* k_cache, void* v_cache, void* q_out,
                             const lbsr_sched_cfg* cfg, void* workspace, size_t ws_bytes, void* out,
                             float* lse_out, void* stream) {
  return decode_step_impl(shape, params, batch, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                          block_table, k_cache, v_cache, q_out, cfg, workspace, ws_bytes, out,
                          lse_out, stream, nullptr, nullptr);
}

lbsr_status lbsr_decode_step_noalloc(const lbsr_shape* shape, const lbsr_params* params,
                                     int32_t batch, const void* q, const void* k, const void* v,
                                     const int32_t* positions, const int32_t* seq_lens,
                                     const void* q_norm_w, const void* k_norm_w,
                                     const int32_t* block_table, void* k_cache, void* v_cache,
                                     void* q_out, const lbsr_sched_cfg* cfg, void* out,
                                     float* lse_out, void* stream) {
  g_last_error[0] = 0;
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  if (l.total > (size_t)LBSR_NOALLOC_SCRATCH_BYTES)
    return fail(LBSR_E_WORKSPACE,
                "this step needs %zu bytes of workspace; the library's scratch holds %zu "
                "(use lbsr_decode_step with a caller workspace)",
                l.total, (size_t)LBSR_NOALLOC_SCRATCH_BYTES);
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  void* ws = nullptr;
  LBSR_CHECK(scratch_of_current_device(&ws));
  return decode_step_impl(shape, params, batch, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                          block_table, k_cache, v_cache, q_out, cfg, ws,
                          (size_t)LBSR_NOALLOC_SCRATCH_BYTES, out, lse_out, stream, nullptr,
                          nullptr);
}

lbsr_status lbsr_decode_step_timed(const lbsr_shape* shape, const lbsr_params* params,
                                   int32_t batch, const void* q, const void* k, const void* v,
                                   const int32_t* positions, const int32_t* seq_lens,
                                   const void* q_norm_w, const void* k_norm_w,
                                   const int32_t* block_table, void* k_cache, void* v_cache,
                                   void* q_out, const lbsr_sched_cfg* cfg, void* workspace,
                                   size_t ws_bytes, void* out, float* lse_out, void* stream,
                                   float* kernel_ms, int64_t* trace) {
  if (!kernel_ms) return fail(LBSR_E_INVALID, "kernel_ms is NULL");
  if (trace && !aligned(trace, 8)) return fail(LBSR_E_INVALID, "trace is not 8-byte aligned");
  return decode_step_impl(shape, params, batch, q, k, v, positions, seq_lens, q_norm_w, k_norm_w,
                          block_table, k_cache, v_cache, q_out, cfg, workspace, ws_bytes, out,
                          lse_out, stream, kernel_ms, trace);
}

lbsr_status lbsr_read_plan(const lbsr_shape* shape, int32_t batch, const lbsr_sched_cfg* cfg,
                           const void* workspace, size_t ws_bytes, lbsr_plan_host* out,
                           int32_t* num_chunks, void* stream) {
  g_last_error[0] = 0;
  if (!out) return fail(LBSR_E_INVALID, "out is NULL");
  lbsr_ws_layout l;
  LBSR_CHECK(compute_layout(shape, batch, cfg, &l));
  LBSR_CHECK(check_workspace(const_cast<void*>(workspace), ws_bytes, l));
  LBSR_CHECK(hip_status(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize"));
  const char* base = (const char*)workspace;
  const struct {
    int32_t* dst;
    size_t off, count;
    const char* what;
  } arrays[] = {
      {out->cu_tiles, l.cu_tiles, (size_t)batch + 1, "cu_tiles"},
      {out->worker_chunk, l.worker_chunk, (size_t)l.num_workers + 1, "worker_chunk"},
      {out->chunks, l.chunks, 4 * (size_t)l.max_chunks, "chunks"},
      {out->seq_chunk, l.seq_chunk, (size_t)batch + 1, "seq_chunk"},
      {out->seq_len_eff, l.seq_len_eff, (size_t)batch, "seq_len_eff"},
  };
  for (const auto& a : arrays)
    if (a.dst)
      LBSR_CHECK(hip_status(hipMemcpy(a.dst, base + a.off, 4 * a.count, hipMemcpyDeviceToHost),
                            a.what));
  if (num_chunks) {
    // the chunk count is the last worker's end: worker_chunk[num_workers]
    LBSR_CHECK(hip_status(hipMemcpy(num_chunks, base + l.worker_chunk + 4 * (size_t)l.num_workers,
                                    4, hipMemcpyDeviceToHost),
                          "chunk count"));
  }
  return LBSR_OK;
}

lbsr_status lbsr_stream_read(const void* buf, size_t bytes, int32_t workgroups, int32_t mode,
                             uint32_t* sink, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(check_ptr(buf, 16, "buf"));
  LBSR_CHECK(check_ptr(sink, 4, "sink"));
  const int64_t blk = lbsr::stream_read_block_bytes();
  if (bytes == 0 || bytes % blk != 0)
    return fail(LBSR_E_INVALID, "bytes (%zu) must be a positive multiple of %lld", bytes,
                (long long)blk);
  if (workgroups < 0 || workgroups > (1 << 20))
    return fail(LBSR_E_INVALID, "workgroups %d outside [0, 2^20]", workgroups);
  if (mode < 0 || mode > 2) return fail(LBSR_E_INVALID, "mode %d is not 0, 1 or 2", mode);
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  const int wg = workgroups ? workgroups : d.cu_count;
  return hip_status(lbsr::launch_stream_read(buf, bytes, wg, mode, sink, (hipStream_t)stream),
                    "stream_read_kernel launch");
}

}  // extern "C"

namespace {

// The row-major form of lbsr_pack_cache / lbsr_unpack_cache: positive
// strides whose byte sizes are multiples of 16, and no two (page, row, head)
// rows overlapping -- with the axes sorted by stride, each stride at least
// the extent of the axes below it (a 128-channel row first).
lbsr_status check_rows(const lbsr_shape* s, int32_t kind, const void* rows, const void* cache,
                       int64_t ps, int64_t ts, int64_t hs) {
  LBSR_CHECK(check_shape(s, 1));
  if (kind != LBSR_CACHE_K && kind != LBSR_CACHE_V)
    return fail(LBSR_E_INVALID, "kind %d is not LBSR_CACHE_K or LBSR_CACHE_V", kind);
  LBSR_CHECK(check_ptr(rows, 16, "rows"));
  LBSR_CHECK(check_ptr(cache, 16, "cache"));
  const int64_t elem = s->kv_dtype == LBSR_KV_BF16 ? 2 : 1;
  const int64_t strides[3] = {ps, ts, hs};
  const int64_t extents[3] = {s->num_pages, LBSR_PAGE_SIZE, s->num_kv_heads};
  const char* names[3] = {"row_page_stride", "row_token_stride", "row_head_stride"};
  // each axis spans at most 2^46 elements, so the reach and the farthest
  // offset below stay far inside int64
  constexpr int64_t kMaxRowElems = (int64_t)1 << 46;
  for (int i = 0; i < 3; ++i) {
    if (strides[i] <= 0 || strides[i] > kMaxRowElems / extents[i] || (strides[i] * elem) % 16)
      return fail(LBSR_E_INVALID,
                  "%s %lld must be positive, span at most 2^46 elements over its %lld entries, "
                  "and be %lld-element aligned",
                  names[i], (long long)strides[i], (long long)extents[i], (long long)(16 / elem));
  }
  int order[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (strides[order[j]] < strides[order[i]]) { const int t = order[i]; order[i] = order[j]; order[j] = t; }
  int64_t reach = LBSR_HEAD_DIM;   // elements one row spans
  for (int i = 0; i < 3; ++i) {
    const int a = order[i];
    if (extents[a] > 1 && strides[a] < reach)
      return fail(LBSR_E_INVALID, "%s %lld overlaps the %lld elements below it", names[a],
                  (long long)strides[a], (long long)reach);
    if (extents[a] > 1) reach = strides[a] * extents[a];
  }
  // the farthest element must be addressable
  const int64_t last = (s->num_pages - 1) * ps + (LBSR_PAGE_SIZE - 1) * ts +
                       (int64_t)(s->num_kv_heads - 1) * hs + LBSR_HEAD_DIM;
  if (last > ((int64_t)1 << 46)) return fail(LBSR_E_INVALID, "row-major extent too large");
  return LBSR_OK;
}

lbsr_status pack_common(bool pack, const lbsr_shape* shape, int32_t kind, const void* src,
                        void* dst, const void* rows, const void* cache, int64_t ps, int64_t ts,
                        int64_t hs, void* stream) {
  g_last_error[0] = 0;
  LBSR_CHECK(check_rows(shape, kind, rows, cache, ps, ts, hs));
  DeviceInfo d;
  LBSR_CHECK(current_device(&d));
  return hip_status(lbsr::launch_pack(shape->kv_dtype == LBSR_KV_FP8_E4M3, kind == LBSR_CACHE_V,
                                      pack, src, dst, shape->num_pages, shape->num_kv_heads,
                                      shape->page_stride, shape->head_stride, ps, ts, hs,
                                      (hipStream_t)stream),
                    pack ? "pack_kernel launch" : "unpack kernel launch");
}

}  // namespace

extern "C" {

lbsr_status lbsr_pack_cache(const lbsr_shape* shape, int32_t kind, const void* rows,
                            int64_t row_page_stride, int64_t row_token_stride,
                            int64_t row_head_stride, void* cache, void* stream) {
  return pack_common(true, shape, kind, rows, cache, rows, cache, row_page_stride,
                     row_token_stride, row_head_stride, stream);
}

lbsr_status lbsr_unpack_cache(const lbsr_shape* shape, int32_t kind, const void* cache,
                              void* rows, int64_t row_page_stride, int64_t row_token_stride,
                              int64_t row_head_stride, void* stream) {
  return pack_common(false, shape, kind, cache, rows, rows, cache, row_page_stride,
                     row_token_stride, row_head_stride, stream);
}

lbsr_status lbsr_read_device_error(const void* workspace, int32_t* code, void* stream) {
  g_last_error[0] = 0;
  if (!code) return fail(LBSR_E_INVALID, "code is NULL");
  LBSR_CHECK(check_ptr(workspace, 256, "workspace"));
  LBSR_CHECK(hip_status(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize"));
  // the error word is the workspace's first array, at offset 0 for every layout
  return hip_status(hipMemcpy(code, workspace, 4, hipMemcpyDeviceToHost), "error word");
}

}  // extern "C"
