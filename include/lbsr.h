/*
 * lbsr -- load-balanced split-KV decode attention with a fused RoPE/QK-Norm
 * prologue, for AMD Instinct MI355X (gfx950).
 *
 * One decode step of grouped-query attention over a paged KV cache:
 *
 *   1. lbsr_rope_norm_kv_write  RoPE + QK-Norm on the new token's q and k and
 *                               the KV-cache write, in one kernel;
 *   2. lbsr_plan                a per-step schedule that deals 64-token tiles
 *                               to workers in proportion to each sequence's
 *                               length (or a static equal split, for
 *                               comparison);
 *   3. lbsr_attention           split attention over the scheduled tiles with
 *                               an online softmax, then a log-sum-exp merge of
 *                               the pieces of sequences that were split;
 *   4. lbsr_decode_step         1 + 2 as one launch (they are independent),
 *                               then 3, on one stream.
 *
 * Sources (titles translated from Korean):
 *   [A] 24-ai.news, "vLLM and Tencent Hunyuan upstream two HPC backends for
 *       NVIDIA Hopper GPUs", sections "Two new HPC backends in the vLLM
 *       ecosystem" (64 q heads, 8 KV heads, head dim 128) and "Why does
 *       dynamic scheduling matter in attention?" (length-proportional
 *       64-token tiles vs static split-KV; fused RoPE + QK-Norm + KV write;
 *       BF16 and FP8).
 *   [B] blog.secrett2633.cloud, "[vllm] Introducing the HPC-Ops attention
 *       backend for high-performance inference in vLLM", intro (FP8 E4M3),
 *       "Code analysis 1" (output dtype passed explicitly), "Code analysis 2"
 *       (the fused op writes a caller-provided output and is entered directly,
 *       so it can be captured in a graph).
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers unless a comment says "host".
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns and allocates every buffer (inputs, outputs, caches,
 *     workspace).  The library allocates no device memory (the one static
 *     device array it holds is the scratch of lbsr_decode_step_noalloc),
 *     keeps no pointer after a call returns, and launches asynchronously on
 *     `stream`; buffers must stay alive until the stream has passed the launch.
 *   - Host-side validation happens before any launch; on failure nothing is
 *     launched, a status is returned and lbsr_last_error() holds a message.
 *   - No entry point synchronises, except lbsr_decode_step_timed (bench) and
 *     the two readers lbsr_read_plan / lbsr_read_device_error (tests, tools).
 *   - Device-side preconditions are checked in the kernels without faulting:
 *     a violating input is clamped or skipped and a bit is OR-ed into the
 *     workspace's sticky error word (see LBSR_DEV_ERR_*).
 *   - Calls on different streams need different workspaces.
 */
#ifndef LBSR_H
#define LBSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBSR_ABI_VERSION 7
#define LBSR_NUM_XCDS 8     /* accelerator complex dies of an MI355X */
#define LBSR_MAX_XCD_WEIGHT 65536
#define LBSR_HEAD_DIM 128
#define LBSR_PAGE_SIZE 64
#define LBSR_TILE_ELEMS (LBSR_HEAD_DIM * LBSR_PAGE_SIZE) /* 8192 elements */

typedef enum {
  LBSR_OK = 0,
  LBSR_E_INVALID = 1,     /* null pointer, size out of range, bad alignment */
  LBSR_E_UNSUPPORTED = 2, /* head_dim != 128, page_size != 64, group > 16, non-gfx950 */
  LBSR_E_WORKSPACE = 3,   /* ws_bytes < the size lbsr_workspace_size reports */
  LBSR_E_HIP = 4          /* a HIP runtime call or launch failed */
} lbsr_status;

typedef enum { LBSR_KV_BF16 = 0, LBSR_KV_FP8_E4M3 = 1 } lbsr_kv_dtype;
typedef enum { LBSR_SCHED_DYNAMIC = 0, LBSR_SCHED_STATIC = 1 } lbsr_sched;
/* Attention output type ([B] "Code analysis 1": the output dtype is passed
 * explicitly).  FP8: out holds OCP E4M3 codes, code = RNE(clamp(o /
 * out_scale, -448, 448)), one byte per element; lse_out stays fp32. */
typedef enum { LBSR_OUT_BF16 = 0, LBSR_OUT_FP8_E4M3 = 1 } lbsr_out_dtype;
/* Arithmetic of Q.K^T with an FP8 cache ([A] "Why does dynamic scheduling
 * matter in attention?": BF16 and FP8 backends; [B] intro: FP8 E4M3).
 * BF16: q stays BF16, the K codes are widened exactly, BF16 matrix cores.
 * FP8_E4M3: q is quantised on load to E4M3 codes RNE(clamp(q * r, -448,
 * 448)) with r = 1/q_scale rounded to fp32 and the product taken in fp32;
 * S = sum over channels of code_q * code_k on FP8 matrix cores (16x16x128),
 * times q_scale * k_scale * sm_scale.  P.V is the same in both. */
typedef enum { LBSR_QK_BF16 = 0, LBSR_QK_FP8_E4M3 = 1 } lbsr_qk_dtype;
/* which pool lbsr_pack_cache / lbsr_unpack_cache convert: K and V tiles
 * order their elements differently */
typedef enum { LBSR_CACHE_K = 0, LBSR_CACHE_V = 1 } lbsr_cache_kind;

/* Sticky device error bits (int32 at lbsr_ws_layout.error_word). */
#define LBSR_DEV_ERR_SEQ_LEN 1   /* seq_len outside [1, max_blocks_per_seq*64]: clamped */
#define LBSR_DEV_ERR_PAGE 2      /* block-table entry outside [0, num_pages): page 0 used */
#define LBSR_DEV_ERR_POSITION 4  /* position outside [0, max_blocks_per_seq*64): write skipped */
#define LBSR_DEV_ERR_QUERY_START 8 /* varlen prefill: q_start range of a sequence malformed
                                      (negative, decreasing, past total_tokens or longer
                                      than shape->tokens_per_seq): sequence skipped */

/*
 * Cache page layout ([A] "Why does dynamic scheduling matter in attention?"
 * fixes only the 64-token tile; the layout is this library's own).
 *
 * The K cache and the V cache are two pools of the same geometry.  Element
 * (page p, KV head g, token row r in [0,64), channel d in [0,128)) lives at
 *     p * page_stride + g * head_stride + tile_offset(r, d)
 * elements from the pool's base.  A tile (one page of one KV head) is 8192
 * contiguous elements: BF16 (16 KiB) or E4M3 codes (8 KiB).  It is stored as
 * 1 KiB fragments of 64 consecutive 16-byte "lanes"; with tb = r/16,
 * kc = (d%32)/8, s = d/32, db = d/16, kv = (r%16)/4, e = 4*(tb%2) + r%4:
 *
 *   K, BF16: 512*(4*tb + s)    + 8*(16*kc + r%16)  + d%8
 *   V, BF16: 512*(2*db + tb/2) + 8*(16*kv + d%16)  + e
 *   K, FP8 : 1024*(2*tb + s/2) + 16*(16*kc + r%16) + 8*(s%2) + d%8
 *   V, FP8 : 1024*db           + 16*(16*kv + d%16) + 8*(tb/2) + e
 *
 * (integer division).  One wave reading one fragment with one 16-byte load
 * per lane gets exactly the operand of one (K) or one (V) matrix-core step;
 * every global read is a contiguous 1 KiB.  Tile t of sequence b is page
 * block_table[b * max_blocks_per_seq + t].
 */

/*
 * Multi-token decode ([A] "Two new HPC backends in the vLLM ecosystem": the
 * model carries a speculative-decoding (MTP) layer, whose drafted tokens are
 * verified by a step with several new tokens per sequence).  With
 * tokens_per_seq = Tq, every array of new tokens gets a token axis after the
 * batch axis -- q, q_out, out [batch][Tq][Hq][128], k, v [batch][Tq][Hkv][128],
 * positions [batch][Tq], lse_out [batch][Tq][Hq] -- and seq_lens[b] counts all
 * Tq of them.  New token j of sequence b sits at position L_b - Tq + j and
 * attends rows [0, L_b - Tq + j]: the cached prefix and new tokens 0..j.
 * The Tq * G queries of one KV head share each KV read: up to 32 of them in
 * one wave (two blocks of 16, one block's accumulator parked in LDS, 16 KiB of
 * LDS per wave); more (up to 64) run as blocks of 16 on neighbouring waves
 * that read the same tiles together.  The merge stages (chunks of a sequence) x
 * (G * Tq) weights in 64 KiB of LDS: a larger product (e.g. 1024 workers
 * with G * Tq = 32) is LBSR_E_UNSUPPORTED.  Tq = 1 is the ordinary step and
 * the layouts reduce to the ones written below.
 */

typedef struct {
  int32_t num_q_heads;        /* Hq >= 1, a multiple of Hkv */
  int32_t num_kv_heads;       /* Hkv >= 1; group G = Hq / Hkv must be <= 16 */
  int32_t head_dim;           /* must be 128 */
  int32_t page_size;          /* must be 64 */
  int32_t kv_dtype;           /* lbsr_kv_dtype */
  int32_t max_blocks_per_seq; /* row stride of block_table, >= 1 */
  int32_t tokens_per_seq;     /* Tq: new tokens per sequence, >= 1 with G * Tq <= 64
                                 (multi-token decode, see below); 1 = one-token step */
  int32_t reserved;           /* must be 0 */
  int64_t num_pages;          /* pages in each pool, >= 1 */
  int64_t page_stride;        /* elements; multiple of 8192; num_pages * page_stride <= 2^46 */
  int64_t head_stride;        /* elements; multiple of 8192; num_kv_heads * head_stride <= 2^46 */
} lbsr_shape;

typedef struct {
  double rope_theta;        /* RoPE base, > 0 (e.g. 1e4) */
  float rms_eps;            /* RMSNorm epsilon, >= 0 (e.g. 1e-6) */
  int32_t norm_before_rope; /* 0: RoPE then RMSNorm (default); 1: RMSNorm then RoPE */
  float k_scale;            /* FP8 cache: value = code * k_scale; > 0; ignored for BF16 */
  float v_scale;            /* FP8 cache: value = code * v_scale; > 0; ignored for BF16 */
  float sm_scale;           /* softmax scale; 0 -> 1/sqrt(128) */
  int32_t out_dtype;        /* lbsr_out_dtype of `out` (0 = BF16) */
  float out_scale;          /* FP8 output: value = code * out_scale; > 0; ignored for BF16 */
  int32_t qk_dtype;         /* lbsr_qk_dtype (0 = BF16); FP8_E4M3 needs an FP8 cache */
  float q_scale;            /* FP8 Q.K^T: q value = code * q_scale; > 0; ignored for BF16 */
} lbsr_params;

/* lbsr_sched_cfg.flags */
#define LBSR_SCHED_FOLD_MERGE 1 /* merge split sequences inside the split-attention
                                 * launch (see lbsr_attention); one new token per
                                 * sequence (tokens_per_seq = 1) only */

typedef struct {
  int32_t sched;         /* lbsr_sched */
  int32_t num_workers;   /* dynamic: P workers in [1, 1024]; 0 -> the device's CU count */
  int32_t static_splits; /* static: S splits per sequence in [1, 1024]; 0 -> max(1, P / batch) */
  int32_t flags;         /* 0, or LBSR_SCHED_FOLD_MERGE */
  /* dynamic only: relative streaming speed of the compute units of each XCD
   * (see lbsr_plan).  All 0 -> every worker gets an equal share; else every
   * entry in [1, LBSR_MAX_XCD_WEIGHT].  Ignored (must be 0) for static. */
  int32_t xcd_weight[LBSR_NUM_XCDS];
} lbsr_sched_cfg;

/* Byte offsets of the arrays inside a workspace (all 256-byte aligned). */
typedef struct {
  size_t error_word;   /* int32: sticky LBSR_DEV_ERR_* bits (the plan clears it) */
  size_t cu_tiles;     /* int32[batch + 1]: prefix sums of ceil(L_b / 64) */
  size_t worker_chunk; /* int32[W + 1]: worker w owns chunks [wc[w], wc[w+1]) */
  size_t chunks;       /* int32[C_max][4]: (sequence, first tile, end tile, worker) */
  size_t seq_chunk;    /* int32[batch + 1]: sequence b owns chunks [sc[b], sc[b+1]) */
  size_t seq_len_eff;  /* int32[batch]: lengths after clamping */
  size_t token_status; /* int32[batch]: prologue error bits per token (decode step) */
  size_t partial_o;    /* float[C_max][Hq][128]: normalised partial outputs */
  size_t partial_lse;  /* float[C_max][Hq]: partial log2-sum-exp (internal) */
  size_t arrivals;     /* int32[batch][Hkv]: chunks of each (sequence, KV head) done, for
                        * LBSR_SCHED_FOLD_MERGE; the plan clears them (internal) */
  size_t total;        /* bytes the workspace needs */
  int32_t num_workers; /* W: workers (= attention workgroups) */
  int32_t max_chunks;  /* C_max = W + batch - 1 (dynamic) or batch * S (static) */
  int32_t static_splits; /* S actually used (static), else 0 */
  int32_t reserved;
} lbsr_ws_layout;

/* ABI version of the loaded library (LBSR_ABI_VERSION). Host only. */
int32_t lbsr_abi_version(void);

/* Text of a status code. Host only; never NULL. */
const char *lbsr_status_string(lbsr_status status);

/* Detail of the last failed call on this thread (empty if none). Host only. */
const char *lbsr_last_error(void);

/* Number of workers the dynamic schedule uses by default on `device`: its
 * compute-unit count (256 on MI355X).  Fails with LBSR_E_UNSUPPORTED if the
 * device is not gfx950. */
lbsr_status lbsr_device_workers(int device, int32_t *out);

/* Workspace layout for a step of `batch` sequences under `cfg`.  Host only
 * when cfg->num_workers > 0 (else it queries the current device).  Like the
 * shape-only "fake" implementation of [B] "Code analysis 2", it needs no
 * device data. */
lbsr_status lbsr_workspace_layout(const lbsr_shape *shape, int32_t batch,
                                  const lbsr_sched_cfg *cfg, lbsr_ws_layout *out);

/* Shorthand: *bytes = lbsr_workspace_layout(...).total. */
lbsr_status lbsr_workspace_size(const lbsr_shape *shape, int32_t batch,
                                const lbsr_sched_cfg *cfg, size_t *bytes);

/*
 * Fused prologue ([A] "Why does dynamic scheduling matter in attention?";
 * [B] "Code analysis 2"): for each new token b at position pos = positions[b]
 *   q_out[b][h] = RMSNorm_wq(RoPE(q[b][h], pos))    for every q head h (BF16)
 *   k'          = RMSNorm_wk(RoPE(k[b][g], pos))    for every KV head g
 * and stores k' and v[b][g] (unchanged) into row pos % 64 of page
 * block_table[b][pos / 64] of the K and V pools: as BF16, or as E4M3 codes
 * RNE(clamp(x / scale, -448, 448)) with k_scale / v_scale.
 * RoPE is rotate-half over all 128 channels: channel i pairs with i + 64 and
 * turns by pos * rope_theta^(-2i/128).  RMSNorm is x / sqrt(mean(x^2) + eps) * w.
 * The arithmetic is fp64; each stored value is rounded once.
 *
 *   q        [batch][Hq][128] BF16           k, v   [batch][Hkv][128] BF16
 *   positions [batch] int32                  q_norm_w, k_norm_w [128] BF16
 *   block_table [batch][max_blocks_per_seq] int32
 *   k_cache, v_cache  pools (layout above)   q_out  [batch][Hq][128] BF16
 *   error_word  nullable int32*: LBSR_DEV_ERR_POSITION / _PAGE are OR-ed in
 * All pointers 16-byte aligned.  A position outside [0, max_blocks*64) or a
 * page outside [0, num_pages) skips that token's cache write (q_out is still
 * written).  q_out may not alias q.
 */
lbsr_status lbsr_rope_norm_kv_write(const lbsr_shape *shape, const lbsr_params *params,
                                    int32_t batch, const void *q, const void *k,
                                    const void *v, const int32_t *positions,
                                    const void *q_norm_w, const void *k_norm_w,
                                    const int32_t *block_table, void *k_cache,
                                    void *v_cache, void *q_out, int32_t *error_word,
                                    void *stream);

/*
 * Tile schedule ([A] "Why does dynamic scheduling matter in attention?").
 * A sequence of length L (the new token included) has n = ceil(L/64) tiles.
 *   dynamic: all tiles laid end to end (T in total); worker w of P owns flat
 *            tiles [floor(T*C(w)/C(P)), floor(T*C(w+1)/C(P))), cut at
 *            sequence ends into chunks, numbered in flat order.  C(w) is the
 *            summed weight of workers 0..w-1.  Unweighted, every worker
 *            weighs 1 and C(w) = w.  Weighted, a worker weighs
 *            xcd_weight[x] of the XCD x it runs on: the attention launch
 *            (workgroup i runs on XCD i mod 8) gives XCD x the contiguous
 *            workers [s(x), s(x) + n(x)), n(x) = ceil((P - x) / 8),
 *            s(x) = n(0) + ... + n(x-1).  MI355X's XCDs stream HBM at
 *            measurably different rates; weights proportional to those
 *            rates let all workers finish together.
 *   static:  every sequence is cut into the same S parts of its own tiles,
 *            [floor(s*n/S), floor((s+1)*n/S)); worker b*S+s; empty parts skipped.
 * Writes the arrays of lbsr_ws_layout into `workspace` (one workgroup, no
 * host sync) and clears the error word.  seq_lens [batch] int32 (device).
 */
lbsr_status lbsr_plan(const lbsr_shape *shape, int32_t batch, const int32_t *seq_lens,
                      const lbsr_sched_cfg *cfg, void *workspace, size_t ws_bytes,
                      void *stream);

/*
 * Split attention + merge over the schedule in `workspace` ([A] "Why does
 * dynamic scheduling matter in attention?": the 64-token tiles dealt out by
 * the schedule are attended on the compute units they were given to, and a
 * split sequence's pieces are merged; [A] "Two new HPC backends in the vLLM
 * ecosystem": q heads grouped over shared KV heads; [B] intro and [A]: BF16
 * or FP8 E4M3 cache).  Run lbsr_plan first with the same shape, batch and
 * cfg.  For sequence b, q head h and
 * KV head g = h / (Hq/Hkv), over the rows j < L_b (with Tq > 1: new token t
 * over the rows j <= L_b - Tq + t, and [b] below reads [b][t]):
 *   out[b][h] = sum_j softmax_j(sm_scale * <q_out[b][h], K_j>) V_j      (BF16)
 *   lse_out[b][h] = ln sum_j exp(sm_scale * <q_out[b][h], K_j>)        (fp32)
 * with K_j = code*k_scale and V_j = code*v_scale for an FP8 cache.  Each
 * chunk is one online-softmax pass over its tiles; a sequence with several
 * chunks is merged by log-sum-exp weights (chunks are summed in a fixed
 * order, so the result is deterministic).
 *   q_out [batch][Hq][128] BF16   out [batch][Hq][128] BF16, or E4M3 codes
 *   (params->out_dtype)           lse_out nullable float[batch][Hq]
 * Rows at or past L_b of a sequence's last page are never used, whatever
 * they hold.  Deterministic.
 * The merge is a second launch by default.  With cfg->flags =
 * LBSR_SCHED_FOLD_MERGE ([A] "Turning the FP8 MoE pipeline into a single
 * execution path" chains kernels to cut the gaps between launches; the same
 * aim applied here) there is one launch:
 * every finished chunk is published with a device-scope fence and counted
 * with a device-scope atomic, and the workgroup (or, when the KV heads do not
 * divide evenly over its waves, the wave) that completes a sequence's count
 * merges its rows in chunk order.  Which one that is varies, the arithmetic
 * does not: results are deterministic either way (but not bit-identical
 * between the two forms).  One new token per sequence; the workspace's
 * arrival counters are cleared by lbsr_plan / the step's plan, and the last
 * arrival of each (sequence, KV head) puts its counter back to zero, so one
 * plan may serve several lbsr_attention calls in stream order.  On MI355X a
 * device-scope release writes back an L2, so this form is slower than two
 * launches except for small, launch-bound batches.
 */
lbsr_status lbsr_attention(const lbsr_shape *shape, const lbsr_params *params, int32_t batch,
                           const void *q_out, const void *k_cache, const void *v_cache,
                           const int32_t *block_table, const lbsr_sched_cfg *cfg,
                           void *workspace, size_t ws_bytes, void *out, float *lse_out,
                           void *stream);

/*
 * One whole decode step ([A] "Why does dynamic scheduling matter in
 * attention?": the prologue fused into one pass, then the per-step
 * length-proportional schedule and the split attention; [B] "Code analysis
 * 2": entered directly with caller-provided outputs, so a HIP graph can
 * capture it) on `stream` (arguments as for the three calls above):
 * the schedule and the prologue in one launch, then split attention and the
 * merge.  Same results as lbsr_plan, lbsr_rope_norm_kv_write and
 * lbsr_attention in turn; the prologue's error bits end up in the
 * workspace's error word.  Requires positions[b] = seq_lens[b] - 1 (with
 * Tq > 1: positions[b][t] = seq_lens[b] - Tq + t) for the new tokens to be
 * part of the attention that follows.
 */
lbsr_status lbsr_decode_step(const lbsr_shape *shape, const lbsr_params *params,
                             int32_t batch, const void *q, const void *k, const void *v,
                             const int32_t *positions, const int32_t *seq_lens,
                             const void *q_norm_w, const void *k_norm_w,
                             const int32_t *block_table, void *k_cache, void *v_cache,
                             void *q_out, const lbsr_sched_cfg *cfg, void *workspace,
                             size_t ws_bytes, void *out, float *lse_out, void *stream);

/*
 * Prefill / chunked-prefill attention ([B] "Why is this good?": the backend
 * is reported on prefill and mixed batches too).  shape->tokens_per_seq = Tq
 * new tokens per sequence, any count up to 2^18 (the decode path's G * Tq <=
 * 64 does not apply); new token t of sequence b (position L_b - Tq + t, its k
 * and v already in the cache) attends rows [0, L_b - Tq + t]:
 *   out[b][t][h]     = sum_j softmax_j(sm_scale * <q_out[b][t][h], K_j>) V_j
 *   lse_out[b][t][h] = ln sum_j exp(sm_scale * <q_out[b][t][h], K_j>)
 * One pass per (sequence, KV head, block of 256/G new tokens; 384/G with FP8
 * scores) over its causal range, each K/V tile read once per block.
 *   q_out [batch][Tq][Hq][128] BF16        seq_lens [batch] int32 (device)
 *   out   [batch][Tq][Hq][128] BF16, or E4M3 codes (params->out_dtype)
 *   lse_out nullable float[batch][Tq][Hq]  error_word nullable int32*
 *   workspace nullable: lbsr_prefill_workspace_size(shape, batch, batch * Tq)
 *     bytes, 256-byte aligned, caller-owned, overwritten by each call.  With
 *     it, a first launch lists the (sequence, block) work items longest first
 *     (grouped by sequence, as the ragged call does) and the attention runs
 *     in that order; without it the grid runs blocks of the last new
 *     tokens first, which is the same order only when every sequence has
 *     the same length.  Workgroups reach compute units in a fixed rotation,
 *     so with unequal lengths the sorted order is much faster (2.1x with one
 *     32K prefix among 1K prefixes).  Results are identical either way.
 * A length outside [Tq, max_blocks*64] is clamped (LBSR_DEV_ERR_SEQ_LEN); a
 * page outside [0, num_pages) reads page 0 (LBSR_DEV_ERR_PAGE).
 */
lbsr_status lbsr_prefill_attention(const lbsr_shape *shape, const lbsr_params *params,
                                   int32_t batch, const void *q_out, const void *k_cache,
                                   const void *v_cache, const int32_t *block_table,
                                   const int32_t *seq_lens, void *workspace, size_t ws_bytes,
                                   void *out, float *lse_out, int32_t *error_word, void *stream);

/*
 * A prefill step: lbsr_rope_norm_kv_write on the Tq new tokens of every
 * sequence (positions[b][t] = seq_lens[b] - Tq + t), then
 * lbsr_prefill_attention, on one stream.  Arguments as for those two calls.
 */
lbsr_status lbsr_prefill_step(const lbsr_shape *shape, const lbsr_params *params,
                              int32_t batch, const void *q, const void *k, const void *v,
                              const int32_t *positions, const int32_t *seq_lens,
                              const void *q_norm_w, const void *k_norm_w,
                              const int32_t *block_table, void *k_cache, void *v_cache,
                              void *q_out, void *workspace, size_t ws_bytes, void *out,
                              float *lse_out, int32_t *error_word, void *stream);

/*
 * Ragged ("varlen") prefill: sequence b has its own count n_b >= 0 of new
 * tokens, as in a chunked-prefill batch of prompts of different lengths
 * ([B] "Why is this good?": prefill and mixed batches).  The new tokens of
 * all sequences are packed along one token axis of total_tokens rows:
 *   q_start  [batch + 1] int32 (device): sequence b's new tokens are rows
 *            [q_start[b], q_start[b+1]) of q_out / out / lse_out; q_start[0]
 *            = 0, non-decreasing, q_start[batch] = total_tokens;
 *   q_out, out [total_tokens][Hq][128]; lse_out nullable [total_tokens][Hq].
 * shape->tokens_per_seq is an upper bound on every n_b.  New token t of
 * sequence b (position L_b - n_b + t) attends rows [0, L_b - n_b + t], as in
 * lbsr_prefill_attention with Tq = n_b.
 * workspace: device memory of lbsr_prefill_workspace_size bytes (required here),
 * 256-byte aligned, caller-owned, overwritten by every call (so calls that
 * share one must be ordered).  A first launch writes there the list of
 * (sequence, block of 256/G new tokens, 384/G with FP8 scores) work items
 * grouped by sequence: the sequences by the rows their longest item attends,
 * longest first, and each sequence's items from its last block (the longest)
 * down, so that blocks
 * which read the same prefix tiles run side by side and share them in L2.
 * The attention launch runs one workgroup per (item, KV head) in that
 * order.  (Workgroups reach compute units in a fixed
 * rotation by index: a grid ordered by sequence, or holding empty blocks,
 * binds CUs to the same few sequences and idles the rest.)  A sequence whose q_start range is
 * malformed (negative, decreasing, past total_tokens, or n_b above the bound)
 * is skipped and flags LBSR_DEV_ERR_QUERY_START; its out rows are not
 * written.  total_tokens = 0 launches nothing.  A mixed batch runs its
 * decoding sequences through lbsr_decode_step (length-balanced split KV) and
 * its prompts through this call, on one stream; one-token sequences are also
 * accepted here, without the split.
 */
lbsr_status lbsr_prefill_attention_varlen(const lbsr_shape *shape, const lbsr_params *params,
                                          int32_t batch, int32_t total_tokens,
                                          const int32_t *q_start, const void *q_out,
                                          const void *k_cache, const void *v_cache,
                                          const int32_t *block_table, const int32_t *seq_lens,
                                          void *workspace, size_t ws_bytes, void *out,
                                          float *lse_out, int32_t *error_word, void *stream);

/* Bytes of a prefill's workspace (its sorted work list): 256 + 8 *
 * (ceil(total_tokens * G / 256) + batch), total_tokens = the packed count of
 * a ragged batch, or batch * tokens_per_seq for the uniform calls (sized for
 * the narrower blocks, so it also holds the FP8-score list).  Host only. */
lbsr_status lbsr_prefill_workspace_size(const lbsr_shape *shape, int32_t batch,
                                        int32_t total_tokens, size_t *bytes);

/*
 * A ragged prefill step: the prologue on all total_tokens packed new tokens
 * (q [total_tokens][Hq][128], k/v [total_tokens][Hkv][128], positions
 * [total_tokens] with positions[q_start[b] + t] = seq_lens[b] - n_b + t; a
 * token's sequence, for its block-table row, is found from q_start), then
 * lbsr_prefill_attention_varlen, on one stream.
 */
lbsr_status lbsr_prefill_step_varlen(const lbsr_shape *shape, const lbsr_params *params,
                                     int32_t batch, int32_t total_tokens,
                                     const int32_t *q_start, const void *q, const void *k,
                                     const void *v, const int32_t *positions,
                                     const int32_t *seq_lens, const void *q_norm_w,
                                     const void *k_norm_w, const int32_t *block_table,
                                     void *k_cache, void *v_cache, void *q_out,
                                     void *workspace, size_t ws_bytes, void *out,
                                     float *lse_out, int32_t *error_word, void *stream);

/*
 * Benchmark helper: lbsr_decode_step with a HIP event recorded on `stream`
 * around each of its three launches (schedule + prologue, split attention,
 * merge, in that order); waits for the stream and writes the three durations
 * in milliseconds to kernel_ms[3] (host).  If `trace` (device, nullable,
 * int64[W][4], W = lbsr_ws_layout.num_workers) is given, the split-attention
 * workgroup of worker w writes {start, end, HW_ID, XCC_ID}: start and end of
 * the device's constant wall clock (hipDeviceAttributeWallClockRate) and the
 * hardware ids of the compute unit it ran on.  Synchronises.  Not for
 * production use.
 */
lbsr_status lbsr_decode_step_timed(const lbsr_shape *shape, const lbsr_params *params,
                                   int32_t batch, const void *q, const void *k,
                                   const void *v, const int32_t *positions,
                                   const int32_t *seq_lens, const void *q_norm_w,
                                   const void *k_norm_w, const int32_t *block_table,
                                   void *k_cache, void *v_cache, void *q_out,
                                   const lbsr_sched_cfg *cfg, void *workspace,
                                   size_t ws_bytes, void *out, float *lse_out,
                                   void *stream, float *kernel_ms, int64_t *trace);

/*
 * The decode step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * lbsr_decode_step with the same arguments minus the workspace.  The
 * workspace lives in a scratch array of LBSR_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on, from its first use there until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); it fails with LBSR_E_WORKSPACE, launching nothing, when
 * the step's workspace (lbsr_workspace_size) would exceed the scratch -- e.g.
 * the 1 x 128K + 31 x 4K batch needs about 9.5 MB, a 4-token step of it about
 * 38 MB.  All calls on one GPU share its scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller.  The schedule launch rewrites every
 * array the later launches read, so nothing carries over between calls.  The
 * device error bits are not readable from outside; callers that need them use
 * lbsr_decode_step with their own workspace.
 */
#define LBSR_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU */
lbsr_status lbsr_decode_step_noalloc(const lbsr_shape *shape, const lbsr_params *params,
                                     int32_t batch, const void *q, const void *k,
                                     const void *v, const int32_t *positions,
                                     const int32_t *seq_lens, const void *q_norm_w,
                                     const void *k_norm_w, const int32_t *block_table,
                                     void *k_cache, void *v_cache, void *q_out,
                                     const lbsr_sched_cfg *cfg, void *out, float *lse_out,
                                     void *stream);

/* Host arrays lbsr_read_plan fills; any may be NULL to skip it.  Sizes come
 * from lbsr_workspace_layout for the same shape, batch and cfg. */
typedef struct {
  int32_t *cu_tiles;     /* [batch + 1] */
  int32_t *worker_chunk; /* [num_workers + 1] */
  int32_t *chunks;       /* [max_chunks][4]; the first worker_chunk[num_workers] rows hold the plan */
  int32_t *seq_chunk;    /* [batch + 1] */
  int32_t *seq_len_eff;  /* [batch] */
} lbsr_plan_host;

/*
 * Test / tool helper: the schedule ([A] "Why does dynamic scheduling matter
 * in attention?") that lbsr_plan or a decode step last wrote into
 * `workspace` (device), copied to the host arrays of *out; *num_chunks (host,
 * nullable) receives the chunk count.  Waits for `stream` first, then copies
 * synchronously.  Validates like lbsr_plan (LBSR_E_WORKSPACE if ws_bytes is
 * too small for the layout).  Not for production paths.
 */
lbsr_status lbsr_read_plan(const lbsr_shape *shape, int32_t batch, const lbsr_sched_cfg *cfg,
                           const void *workspace, size_t ws_bytes, lbsr_plan_host *out,
                           int32_t *num_chunks, void *stream);

/*
 * Test / tool helper: the sticky LBSR_DEV_ERR_* bits of a decode workspace
 * (its first int32, the error word of every layout) into *code (host).  Waits
 * for `stream` first.  The device-side checks of a step ([A] "Why does
 * dynamic scheduling matter in attention?": lengths, pages and positions the
 * schedule and the cache write rely on) report here instead of faulting.
 */
lbsr_status lbsr_read_device_error(const void *workspace, int32_t *code, void *stream);

/*
 * Benchmark helper, not an operation of the method: reads `bytes` (a positive
 * multiple of 32 KiB) of device memory at `buf` (16-byte aligned) with
 * non-temporal 16-byte loads, in `workgroups` workgroups of 8 waves (0 -> the
 * device's CU count), and writes one checksum word per workgroup to `sink`
 * (device, uint32[workgroups]).  mode 0 reads the way the split-attention
 * kernel reads K/V tiles: one 32 KiB burst per wave, the 8 waves meeting at a
 * barrier after each burst is issued.  mode 1 is a plain sweep: every thread
 * keeps 8 loads in flight, one grid-width apart, with no barriers.  mode 2 is
 * mode 0 with 16 KiB bursts loaded straight into LDS (global-to-LDS loads,
 * 128 KiB of LDS per workgroup) and read back from there.  The best rate over
 * modes and grid sizes is the streaming ceiling the split kernel's bandwidth
 * is reported against.  Asynchronous on `stream`.
 */
lbsr_status lbsr_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t mode,
                             uint32_t *sink, void *stream);

/*
 * Cache layout conversion, for callers whose paged cache is a plain row-major
 * array.  [A] "Why does dynamic scheduling matter in attention?" fixes the
 * 64-token page as the unit the cache is read in; the element order inside a
 * page (the "cache page layout" above) is this library's own, so such a
 * caller repacks its pool once with lbsr_pack_cache and can read it back with
 * lbsr_unpack_cache.
 *
 * The row-major form: element (page p, token row r in [0,64), KV head g,
 * channel d) at  p * row_page_stride + r * row_token_stride
 *                + g * row_head_stride + d  elements from `rows`.
 * Channels are contiguous; any order of the other three axes works (e.g.
 * token-major [pages][64][Hkv][128]: strides 64*Hkv*128, Hkv*128, 128;
 * head-major [pages][Hkv][64][128]: Hkv*64*128, 128, 64*128).  The strides
 * must be positive, their byte sizes multiples of 16, each axis may span at
 * most 2^46 elements (stride x entries), and no two (page, row, head) rows
 * may overlap (sorted by stride, each stride at least the extent of the axes
 * below it); else LBSR_E_INVALID.
 *
 * `cache` is a pool of the library's layout with shape->num_pages pages,
 * shape->page_stride and shape->head_stride; every (page, KV head) tile of it
 * is converted.  The element type is shape->kv_dtype: BF16, or E4M3 codes
 * moved as bytes (no scale is applied: the codes must already be those of
 * the cache's per-tensor scale).  `kind` (lbsr_cache_kind) selects K or V.
 * Device pointers, 16-byte aligned; `rows` and `cache` must not overlap.
 * The shape is validated as for the other calls (with a batch of 1).
 * Asynchronous on `stream`; the library allocates nothing.
 */
lbsr_status lbsr_pack_cache(const lbsr_shape *shape, int32_t kind, const void *rows,
                            int64_t row_page_stride, int64_t row_token_stride,
                            int64_t row_head_stride, void *cache, void *stream);

/* The inverse of lbsr_pack_cache: every tile of `cache` written back to the
 * row-major `rows` (same arguments and checks). */
lbsr_status lbsr_unpack_cache(const lbsr_shape *shape, int32_t kind, const void *cache,
                              void *rows, int64_t row_page_stride, int64_t row_token_stride,
                              int64_t row_head_stride, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LBSR_H */
