/*
 * kvsel.h -- C ABI of the attention-score KV selection and compaction library
 * (libkvsel.so, HIP kernels for gfx950 / MI355X).
 *
 * One layer-end step of an observation-window KV eviction method, as the
 * three calls of the path:
 *
 *   kvsel_score    observation-window attention scores, reduced over the
 *                  window queries and the GQA group, then max-pooled
 *   kvsel_select   top-`budget` candidate positions per KV head, plus the
 *                  always-kept sinks and observation window
 *   kvsel_compact  gather of the kept K/V rows into a compact cache
 *
 * and around them:
 *   kvsel_layer_end, kvsel_layer_end_stream, kvsel_layer_end_adaptive
 *                  the whole step in one call (radix select over the score
 *                  vector; streaming top-k inside pass 2; one head-adaptive
 *                  budget per sequence into a flattened cache)
 *   kvsel_select_compact, kvsel_select_adaptive, kvsel_compact_flat
 *                  select and gather in one call; the head-adaptive select
 *                  and its flattened gather
 *   kvsel_route_tiers, kvsel_qevict_step
 *                  contiguous-window routing into full / low-bit / evicted
 *                  tiers (one shot; repeated over decode steps with a
 *                  backing store)
 *   kvsel_kara_score, kvsel_kara_select, kvsel_kara_keep
 *                  decode-window compression by bidirectional scores and
 *                  chunked selection
 *   kvsel_score_static  kvsel_score without a workspace argument
 *   kvsel_timing_start, kvsel_timing_read  per-kernel device timing
 *
 * Sources (web pages this library implements; title, then section/equation):
 *   [TideKV] "TideKV: Delayed KV Eviction via Layer-Wise Chunked Prefill for
 *            Memory-Efficient Long-Context LLM Inference", Section 4.2
 *            (Eqs. 4-8), Algorithm 2 (LayerEndCompress), Algorithm 1,
 *            Section 4.1 (head-adaptive budgets).
 *   [QEvict] "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-
 *            Robust Long-Context Decoding", Sections 4.1-4.3, Appendix A.
 *   [Kara]   "Kara: Efficient Reasoning LLM Serving via Sliding-Window KV
 *            Cache Compression", Section 3 (Eqs. 4-8).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Shapes use: Bt batch, Hq query heads, Hkv KV heads (G = Hq/Hkv), D head
 *    dimension, S prompt length, W observation window, n_sink leading
 *    mandatory positions.  All tensors are dense, row-major, contiguous.
 *      q_obs   [Bt, Hq,  W, D]   element type `dtype`
 *      k, v    [Bt, Hkv, S, D]   element type `dtype`
 *      scores  [Bt, Hkv, S]      float32
 *      idx     [Bt, Hkv, n_keep] int32, n_keep = budget + n_sink + W
 *      k_out   [Bt, Hkv, n_keep, D]
 *    Query head h reads KV head floor(h / G).
 *  - Every pointer argument is a DEVICE pointer (hipMalloc'd or equivalent)
 *    unless stated otherwise and must be 16-byte aligned.  The caller owns all
 *    buffers; the library never allocates or frees device memory.  Scratch
 *    memory is passed in as `ws` with a size from the matching *_workspace()
 *    query (kvsel_score_static alone uses a static array inside the library).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; no call synchronises the host or reads device memory back.
 *  - Every precondition is checked before anything is enqueued.  A failed check
 *    returns a status and enqueues nothing; checks never touch the GPU, so the
 *    argument validation also runs on a machine without a GPU.  A failed
 *    kernel launch returns KVSEL_ERR_DEVICE.  No C++ exception crosses the ABI.
 *  - Output buffers must not overlap inputs or each other.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    must use different workspaces and outputs.
 *  - Debugging switches, read from the environment at every call:
 *    KVSEL_VALIDATE_ONLY=1 makes a call return after its checks without
 *    enqueuing anything; KVSEL_SYNC=1 makes a call wait for its stream and
 *    report a device error (a failed or faulting kernel) as KVSEL_ERR_DEVICE;
 *    KVSEL_SCORE_COMBINE=1 makes the score passes always merge the row
 *    statistics in a separate launch (small problems otherwise merge them
 *    inside the second pass; both give the same bits).
 *  - The library keeps no state between calls, except the optional kernel
 *    timing of kvsel_timing_start (off unless turned on) and the static
 *    scratch array of kvsel_score_static.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSEL_OK = 0,
  KVSEL_ERR_ARG = 1,          /* bad shape, null or misaligned pointer, bad enum */
  KVSEL_ERR_BUDGET = 2,       /* budget outside [0, S - W - n_sink] */
  KVSEL_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the workspace query */
  KVSEL_ERR_UNSUPPORTED = 4,  /* valid but not built for these sizes (head_dim other
                                 than 64/128, and the limits each call states) */
  KVSEL_ERR_DEVICE = 5        /* a HIP launch reported an error */
} kvsel_status;

typedef enum { KVSEL_BF16 = 0, KVSEL_F32 = 1 } kvsel_dtype;

/* Shape of one layer-end selection problem. */
typedef struct {
  int32_t batch;       /* Bt >= 1 */
  int32_t n_q_heads;   /* Hq >= 1, multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t seq_len;     /* S >= 1: keys in the layer's full prompt KV */
  int32_t obs_window;  /* W, 1 <= W <= S: observation queries; with causal=1
                          also the last W key positions, always kept */
  int32_t n_sink;      /* leading positions always kept, 0 <= n_sink <= S - W */
  int32_t causal;      /* 1: query q (0-based) sits at position S-W+q and sees
                          keys <= S-W+q (TideKV Eq. 4 causal mask);
                          0: queries follow the cache and see every key */
  int32_t dtype;       /* kvsel_dtype of q_obs, k and v */
  float scale;         /* logit scale; 0 selects 1/sqrt(head_dim) (Eq. 4) */
} kvsel_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* kvsel_status_str(kvsel_status s);

/* Bytes of scratch kvsel_score needs for `desc` (0 on an invalid desc). */
size_t kvsel_score_workspace(const kvsel_desc* desc);

/*
 * kvsel_score -- per-KV-head key importance, TideKV Section 4.2.
 *
 * For each (b, query head h, window query q) the logits are
 *   l[i] = scale * <q_obs[b,h,q,:], k[b,floor(h/G),i,:]>          (Eq. 4)
 * (-inf past the query's causal position when causal=1), normalised with the
 * row's log-sum-exp found in a first streaming pass over the keys
 * (Eqs. 5-6) and recomputed in a second pass (Eq. 7, left):
 *   a[i] = exp(l[i] - M) / Z.
 * raw_scores[b,hk,i] = sum over the G query heads of KV head hk and the W
 * queries of a[i]  (Eq. 7, right, with unit pooling weights; a sum, so each
 * head's row sums to G*W).
 * pooled[b,hk,i] = max of raw_scores over positions j with |j - i| <= h,
 * h = (pool_kernel-1)/2, and j in the candidate range C = [n_sink, S-W),
 * for i in C; 0 outside C (the "pool to p_i" step of Algorithm 2, read as a
 * stride-1 1-D max filter that does not reach into the mandatory ranges).
 *
 *   q_obs       [Bt,Hq,W,D] dtype, device
 *   k           [Bt,Hkv,S,D] dtype, device
 *   raw_scores  [Bt,Hkv,S] float32, device, may be NULL (then kept in ws)
 *   pooled      [Bt,Hkv,S] float32, device; may be NULL when raw_scores is
 *               given (callers that rank the raw scores themselves, as the
 *               decode-time window routers do, skip the max filter)
 *   pool_kernel odd, >= 1
 *   ws          device scratch of >= kvsel_score_workspace(desc) bytes
 *               (may be NULL when that size is 0)
 * Errors: KVSEL_ERR_ARG (shape, pointer, both outputs NULL, pool_kernel even
 *         or < 1), KVSEL_ERR_UNSUPPORTED (head_dim), KVSEL_ERR_WORKSPACE,
 *         KVSEL_ERR_DEVICE.
 * Numerics: bf16 or fp32 inputs, fp32 products and sums; the result does
 * not depend on how the keys are blocked; repeated calls are bitwise equal.
 * Kernels: unmasked bf16 problems of at most 512 keys in whole 32-key tiles
 * with at least 256 query rows per KV head run both passes in one launch per
 * KV head, its keys held on chip; others run the two passes over key chunks.
 */
kvsel_status kvsel_score(const kvsel_desc* desc, const void* q_obs, const void* k,
                         float* raw_scores, float* pooled, int32_t pool_kernel,
                         void* ws, size_t ws_bytes, void* stream);

/* Bytes of scratch kvsel_select needs for `desc` and `budget` (0 when rows
 * have up to about 16384 candidates and fit the single-workgroup kernel, or on
 * invalid arguments).  Long rows use a sliced multi-workgroup radix select whose
 * scratch is about 8 bytes per candidate position plus per-slice counters. */
size_t kvsel_select_workspace(const kvsel_desc* desc, int32_t budget);

/*
 * kvsel_select -- retained set R per (b, KV head), TideKV Eq. (8).
 *
 * R = Top_budget{ pooled[i] : i in [n_sink, S-W) }  U  [0, n_sink)  U  [S-W, S),
 * candidates ordered by (score descending, position ascending), so equal
 * scores keep the lowest positions.  The mandatory set is always kept and
 * `budget` counts only the non-mandatory picks: |R| = budget + n_sink + W,
 * which is TideKV's K_l with the window counted inside the budget.
 * idx[b,hk,:] receives R in ascending position order (int32).
 *
 *   pooled  [Bt,Hkv,S] float32, device; every candidate value must be a
 *           finite number >= 0 (as kvsel_score produces)
 *   budget  0 <= budget <= S - W - n_sink, else KVSEL_ERR_BUDGET
 *   idx     [Bt,Hkv,budget+n_sink+W] int32, device
 * Selection is exact: the budget-th largest value is found bit for bit by a
 * radix select over the fp32 bit patterns.
 */
kvsel_status kvsel_select(const kvsel_desc* desc, const float* pooled, int32_t budget,
                          int32_t* idx, void* ws, size_t ws_bytes, void* stream);
/* (kvsel_select: ws is device scratch of >= kvsel_select_workspace(desc,
 * budget) bytes, may be NULL when that is 0; else KVSEL_ERR_WORKSPACE.) */

/* Bytes of scratch kvsel_select_adaptive needs: 0 when a sequence has up to about
 * 16384 candidates (one workgroup per sequence), when total_budget is 0, or
 * on invalid arguments; otherwise about 8 bytes per candidate position of
 * every KV head plus per-slice counters. */
size_t kvsel_select_adaptive_workspace(const kvsel_desc* desc, int32_t total_budget);

/*
 * kvsel_select_adaptive -- head-adaptive retained sets in a flattened layout
 * with per-head offsets (TideKV Section 4.1: a head-adaptive budget gives a
 * variable-length cache, flattened, with per-head offsets; Eq. (8) applied to
 * all KV heads of a sequence at once).
 *
 * For each sequence b the candidates are the pairs (hk, i), i in
 * [n_sink, S-W), over all Hkv heads; the total_budget largest pooled scores
 * are picked, ordered by (score descending, head ascending, position
 * ascending).  There is no per-head floor beyond the mandatory set: every
 * head keeps its sinks [0, n_sink) and its window [S-W, S).
 *
 *   pooled    [Bt,Hkv,S] float32, device; candidates finite and >= 0
 *   total_budget  0 <= total_budget <= Hkv*(S-W-n_sink), else
 *             KVSEL_ERR_BUDGET (callers counting the mandatory rows inside
 *             a per-sequence budget pass that budget minus Hkv*(n_sink+W))
 *   idx       [Bt, n_keep] int32 out, n_keep = Hkv*(n_sink+W) + total_budget:
 *             head hk's positions, ascending, in rows
 *             [head_off[b,hk], head_off[b,hk+1])
 *   head_off  [Bt, Hkv+1] int32 out; head_off[b,0] = 0, head_off[b,Hkv] = n_keep
 *   ws        device scratch of >= kvsel_select_adaptive_workspace bytes
 * Needs Hkv <= 64, Hkv*S < 2^31 and, when a sequence has more than 16384
 * candidates, at most 2048 slices of 4096 candidates per sequence
 * (KVSEL_ERR_UNSUPPORTED otherwise).  Selection is exact as in kvsel_select.
 */
kvsel_status kvsel_select_adaptive(const kvsel_desc* desc, const float* pooled,
                                   int32_t total_budget, int32_t* idx, int32_t* head_off,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_compact_flat -- GATHER into the flattened per-head-offset layout:
 * for head_off[b,hk] <= r < head_off[b,hk+1],
 * k_out[b,r,:] = k[b,hk,idx[b,r],:], and the same for v, byte for byte.
 *
 *   k, v         [Bt,Hkv,S,D] dtype, device
 *   idx          [Bt,n_keep] int32, head_off [Bt,Hkv+1] int32, device (as
 *                written by kvsel_select_adaptive)
 *   n_keep       0 <= n_keep <= Hkv*S
 *   k_out, v_out [Bt,n_keep,D] dtype, device
 * A row whose index is outside [0, S) is written as zeros; a row below
 * head_off[b,0] or at/after head_off[b,Hkv] is taken from the first or the
 * last head, so malformed offsets never read out of bounds.  v may be NULL
 * together with v_out.
 */
kvsel_status kvsel_compact_flat(const kvsel_desc* desc, const void* k, const void* v,
                                const int32_t* idx, const int32_t* head_off, int32_t n_keep,
                                void* k_out, void* v_out, void* stream);

/*
 * kvsel_compact -- GATHER of Algorithm 2: k_out[b,hk,r,:] = k[b,hk,idx[b,hk,r],:]
 * and the same for v, byte for byte.  The position metadata of the compact
 * cache is idx itself (absolute positions, TideKV Section 5 cache manager).
 *
 *   k, v         [Bt,Hkv,S,D] dtype, device
 *   idx          [Bt,Hkv,n_keep] int32, device
 *   n_keep       >= 0
 *   k_out, v_out [Bt,Hkv,n_keep,D] dtype, device
 * An index outside [0, S) yields an all-zero row (never an out-of-bounds
 * read).  v may be NULL together with v_out to gather K only.
 */
kvsel_status kvsel_compact(const kvsel_desc* desc, const void* k, const void* v,
                           const int32_t* idx, int32_t n_keep, void* k_out, void* v_out,
                           void* stream);

/*
 * kvsel_select_compact -- kvsel_select followed by kvsel_compact with
 * n_keep = budget + n_sink + W (Eq. 8, then Algorithm 2's GATHER), in one
 * launch when a KV head's candidates fit one workgroup and n_keep <= 4096
 * (every other shape runs the two steps in order).  The outputs are exactly
 * those of the two calls: idx as kvsel_select writes it, and k_out, v_out as
 * kvsel_compact writes them from that idx.
 *
 *   pooled       [Bt,Hkv,S] float32, device (kvsel_score)
 *   idx          [Bt,Hkv,budget+n_sink+W] int32 out, device
 *   k, v         [Bt,Hkv,S,D] dtype, device (v may be NULL with v_out)
 *   k_out, v_out [Bt,Hkv,budget+n_sink+W,D] dtype out, device
 *   ws           device scratch of >= kvsel_select_workspace(desc, budget)
 * Errors: those of kvsel_select and kvsel_compact.
 */
kvsel_status kvsel_select_compact(const kvsel_desc* desc, const float* pooled, int32_t budget,
                                  int32_t* idx, const void* k, const void* v, void* k_out,
                                  void* v_out, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_layer_end -- TideKV Algorithm 2 (LayerEndCompress) in one call:
 * kvsel_score, then kvsel_select_compact, with exactly their results
 * (raw and pooled scores, idx, k_out, v_out as those calls define them).
 * For long rows the max filter, the selection and the gather run fused
 * behind the two score passes (fewer kernel launches, the same bits).
 *
 *   q_obs        [Bt,Hq,W,D] dtype, device
 *   k, v         [Bt,Hkv,S,D] dtype, device (v may be NULL together with v_out)
 *   budget       0 <= budget <= S - W - n_sink, else KVSEL_ERR_BUDGET
 *   pool_kernel  odd, >= 1
 *   raw_scores   [Bt,Hkv,S] float32 out, device, may be NULL (kept in ws)
 *   pooled       [Bt,Hkv,S] float32 out, device, may be NULL (kept in ws)
 *   idx          [Bt,Hkv,budget+n_sink+W] int32 out, device, ascending
 *   k_out, v_out [Bt,Hkv,budget+n_sink+W,D] dtype out, device
 *   ws           device scratch of >= kvsel_layer_end_workspace(desc, budget)
 *                bytes (computed for pooled == NULL, the larger case)
 * Errors: those of kvsel_score and kvsel_select_compact.
 */
size_t kvsel_layer_end_workspace(const kvsel_desc* desc, int32_t budget);
kvsel_status kvsel_layer_end(const kvsel_desc* desc, const void* q_obs, const void* k,
                             const void* v, int32_t budget, int32_t pool_kernel,
                             float* raw_scores, float* pooled, int32_t* idx, void* k_out,
                             void* v_out, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_layer_end_adaptive -- TideKV Algorithm 2 with the head-adaptive
 * budget of Section 4.1 in one call: kvsel_score, then kvsel_select_adaptive,
 * then kvsel_compact_flat with n_keep = Hkv*(n_sink+W) + total_budget, with
 * exactly their results (raw and pooled scores, idx, head_off, k_out, v_out
 * as those calls define them).  When a sequence's candidates span at most
 * 1024 slices of 4096, the max filter runs fused with the selection's first
 * histogram behind the two score passes (fewer launches, the same bits).
 *
 *   q_obs         [Bt,Hq,W,D] dtype, device
 *   k, v          [Bt,Hkv,S,D] dtype, device (v may be NULL with v_out)
 *   total_budget  0 <= total_budget <= Hkv*(S-W-n_sink), else KVSEL_ERR_BUDGET
 *   pool_kernel   odd, >= 1
 *   raw_scores    [Bt,Hkv,S] float32 out, device, may be NULL (kept in ws)
 *   pooled        [Bt,Hkv,S] float32 out, device, may be NULL (kept in ws)
 *   idx           [Bt,n_keep] int32 out; head_off [Bt,Hkv+1] int32 out
 *   k_out, v_out  [Bt,n_keep,D] dtype out, device
 *   ws            device scratch of >= kvsel_layer_end_adaptive_workspace(desc,
 *                 total_budget) bytes (computed for pooled == NULL)
 * Errors: those of kvsel_score, kvsel_select_adaptive and kvsel_compact_flat.
 */
size_t kvsel_layer_end_adaptive_workspace(const kvsel_desc* desc, int32_t total_budget);
kvsel_status kvsel_layer_end_adaptive(const kvsel_desc* desc, const void* q_obs, const void* k,
                                      const void* v, int32_t total_budget, int32_t pool_kernel,
                                      float* raw_scores, float* pooled, int32_t* idx,
                                      int32_t* head_off, void* k_out, void* v_out, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * kvsel_layer_end_stream -- TideKV Algorithm 2 with its streaming top-k: the
 * top candidates are kept while pass 2 streams over the keys (Section 4.2,
 * the heap of pass 2, and its temporary-memory bound), so no per-key score
 * vector is formed.  Each workgroup of pass 2 pools its key chunk in LDS and
 * keeps the chunk's top-`budget` candidates; a selection over the per-row
 * candidate lists picks the final top-`budget`.  idx, k_out and v_out are
 * exactly those of kvsel_layer_end (the same scores, the same order of
 * ties); raw and pooled scores are not returned.
 *
 *   arguments as kvsel_layer_end without raw_scores / pooled
 *   ws  device scratch of >= kvsel_layer_end_stream_workspace(desc, budget,
 *       pool_kernel) bytes: O(rows x chunks x budget) for the candidate
 *       lists, independent of S while the chunk count (set by the size of
 *       the GPU) is fixed
 * Supported: bf16 prompts of 4096 keys or more with G*W <= 320 query rows
 * per KV head, key chunks of at most 16384 keys, pool_kernel <= 129;
 * otherwise KVSEL_ERR_UNSUPPORTED (the workspace query returns 0).
 */
size_t kvsel_layer_end_stream_workspace(const kvsel_desc* desc, int32_t budget,
                                        int32_t pool_kernel);
kvsel_status kvsel_layer_end_stream(const kvsel_desc* desc, const void* q_obs, const void* k,
                                    const void* v, int32_t budget, int32_t pool_kernel,
                                    int32_t* idx, void* k_out, void* v_out, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Kara decode-window compression (Kara, "Kara: Efficient Reasoning LLM
 * Serving via Sliding-Window KV Cache Compression", Section 3).  A window of
 * `window` recent tokens per (sequence, KV head); its last `buffer` tokens
 * (U) are never compressed; the first n = window - buffer are the
 * compressible region.
 */
typedef struct {
  int32_t batch;       /* Bt >= 1 */
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t window;      /* |W| >= 2 */
  int32_t buffer;      /* |U|, 0 <= buffer < window */
  int32_t keep;        /* size of I, ceil(r * (window - buffer)) for ratio r (Eq. 5) */
  int32_t gamma;       /* maximum chunk length, >= 1 (Eq. 7) */
  int32_t alpha;       /* chunk budget: extra positions added, >= 0, any int32 (Eq. 7,
                          fill-up); when fewer free positions remain, all are added */
  int32_t dtype;       /* kvsel_dtype of q and k */
  float scale;         /* logit scale; 0 => 1/sqrt(head_dim) */
} kvsel_kara_desc;

/* Bytes of scratch kvsel_kara_score needs (0 on invalid arguments). */
size_t kvsel_kara_score_workspace(const kvsel_kara_desc* desc);

/*
 * kvsel_kara_score -- sliding-window bidirectional importance (Kara Eq. 4):
 * scores[b,hk,j] = sum over the window queries i of the G query heads of KV
 * head hk of softmax_j'(<Q_i, K_j'> * scale) at j, the softmax running over
 * the compressible keys j' < n only, with no causal mask.
 *
 *   q_win   [Bt,Hq,window,D] dtype, device: the queries of every window token
 *   k_win   [Bt,Hkv,window,D] dtype, device: the window's keys (rows >= n,
 *           the buffer, are not read)
 *   scores  [Bt,Hkv,n] float32 out, device
 * Same kernels and numerics as kvsel_score on the same shape (fp32 products
 * and sums); a window of n = window - buffer keys in whole 32-key tiles, up
 * to 512, with G*window >= 256 query rows is scored in one launch per KV head.
 */
kvsel_status kvsel_kara_score(const kvsel_kara_desc* desc, const void* q_win, const void* k_win,
                              float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_kara_select -- Token2Chunk selection (Kara Eqs. 5-8 and the fill-up
 * rule after them).  Per (b, hk): I = the `keep` highest scores (ties to the
 * lower position); for consecutive members of I (ascending) at most gamma
 * apart, chunk k scores (A[I[k]] + A[I[k+1]]) * (I[k+1] - I[k] - 1) in fp32;
 * the floor(alpha/gamma) best chunks (ties to the lower k) add their interior
 * positions; then, while fewer than alpha positions were added, the best
 * remaining positions by score are added (ties to the lower position).
 *
 *   scores  [Bt,Hkv,n] float32, device (kvsel_kara_score), finite
 *   idx     [Bt,Hkv,min(n, keep+alpha) + buffer] int32 out, device: the kept
 *           compressible positions ascending, then n..window-1 (the buffer);
 *           window-relative, so kvsel_compact with seq_len = window gathers
 *           the compressed window
 * n = window - buffer must be at most 2048 (KVSEL_ERR_UNSUPPORTED).
 */
kvsel_status kvsel_kara_select(const kvsel_kara_desc* desc, const float* scores, int32_t* idx,
                               void* stream);

/*
 * kvsel_kara_keep -- |I| of Kara Eq. (5) for a retention ratio given as the
 * fraction r = ratio_num / ratio_den: ceil(r * (window - buffer)), computed
 * exactly in integer arithmetic (no rounding of r).  This is the `keep`
 * field of kvsel_kara_desc.  Returns -1 when window < 2, buffer is outside
 * [0, window), ratio_den < 1, or ratio_num is outside [0, ratio_den].
 * Host-only; touches no device state.
 */
int32_t kvsel_kara_keep(int32_t window, int32_t buffer, int32_t ratio_num, int32_t ratio_den);

/* Shape of a window-tier routing problem (QEvict Sections 4.1-4.3). */
typedef struct {
  int32_t batch;       /* Bt >= 1 */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t seq_len;     /* S, a multiple of win */
  int32_t win;         /* tokens per window and per int4 group: 64 */
  int32_t n_full;      /* windows kept in the full-precision tier */
  int32_t n_quant;     /* windows kept in the int4 tier; n_full + n_quant <= S/win */
  int32_t dtype;       /* kvsel_dtype of k, v: KVSEL_BF16 only */
} kvsel_tier_desc;

/* Bytes of scratch kvsel_route_tiers needs. */
size_t kvsel_route_tiers_workspace(const kvsel_tier_desc* desc);

/*
 * kvsel_route_tiers -- QEvict cumulative window scoring and three-tier routing.
 *
 * Window j of (b, hk) covers tokens [j*win, (j+1)*win); its score is the sum
 * of token_scores over the window (Section 4.2, cumulative attention).
 * Windows are ranked by (score descending, index ascending); ranks
 * [0, n_full) go to the full tier (0), the next n_quant to the int4 tier (1),
 * the rest are evicted (2) (Section 4.3, routing by rank under tier
 * capacities).  Within each tier windows keep ascending index order.
 *
 * int4 rule for one group = one channel c of one window, K and V separately
 * (asymmetric codes, Section 4.3; formula is this library's reading):
 *   lo = min x, hi = max x, scale = (hi - lo) / 15  (fp32, IEEE division)
 *   code = 0 if scale == 0 else clamp(rint((x - lo) / scale), 0, 15),
 *   rint rounding half to even; packed two per byte, even channel in the
 *   low nibble.  Dequantisation: x' = bf16_rne(lo + code * scale), with the
 *   product and the sum each rounded to fp32 (no fused multiply-add).
 *
 *   token_scores [Bt,Hkv,S] float32 (e.g. kvsel_score raw scores)
 *   k, v         [Bt,Hkv,S,D] bf16
 *   tier         [Bt,Hkv,S/win] int8 out
 *   win_rank     [Bt,Hkv,S/win] int32 out (0 = highest score)
 *   k_full,v_full [Bt,Hkv,n_full*win,D] bf16 out: full-tier windows copied
 *   k_codes,v_codes [Bt,Hkv,n_quant,win,D/2] uint8 out: packed codes
 *   k_meta,v_meta   [Bt,Hkv,n_quant,D,2] float32 out: (lo, scale)
 *   promote      [Bt,Hkv,n_promote] int32: slots in [0, n_quant) of the int4
 *                tier (its ascending window order) to promote; may be NULL
 *                when n_promote == 0
 *   k_prom,v_prom [Bt,Hkv,n_promote*win,D] bf16 out: dequantised windows
 * A promote slot outside [0, n_quant) yields all-zero rows.
 * Scores closer than fp32 rounding may rank differently from an exact sum.
 */
kvsel_status kvsel_route_tiers(const kvsel_tier_desc* desc, const float* token_scores,
                               const void* k, const void* v, int8_t* tier, int32_t* win_rank,
                               void* k_full, void* v_full, uint8_t* k_codes, uint8_t* v_codes,
                               float* k_meta, float* v_meta, const int32_t* promote,
                               int32_t n_promote, void* k_prom, void* v_prom,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Repeated recoverable routing (QEvict, "Recoverable Quantized KV Eviction for
 * Attention-Drift-Robust Long-Context Decoding": Sections 4.1-4.3 and
 * Appendix A, repeated every Omega decode tokens as in Section 4.2, with the
 * persistent quantised backing store of Section 1).  Per (sequence, KV head)
 * the cache rows [n_sink, n_sink + 64*nW) are cut into nW = floor((seq_len -
 * n_sink - n_recent) / 64) windows; the sinks, the recent tokens and a
 * partial window before them are protected (never routed, never changed).
 */
typedef struct {
  int32_t batch;        /* Bt >= 1 */
  int32_t n_kv_heads;   /* Hkv >= 1, Bt*Hkv <= 65535 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t seq_len;      /* tokens currently in the cache (<= capacity) */
  int32_t capacity;     /* cache rows per (sequence, KV head) in k, v */
  int32_t max_windows;  /* window slots per (sequence, KV head) in the state (<= 4096) */
  int32_t win;          /* tokens per window: 64 */
  int32_t n_sink;       /* protected leading tokens (QEvict's default: 5) */
  int32_t n_recent;     /* protected trailing tokens */
  int32_t n_full;       /* full-precision window capacity */
  int32_t n_quant;      /* quantised window capacity */
  int32_t bits;         /* 2 (QEvict's default tier) or 4 */
  int32_t dtype;        /* kvsel_dtype of k, v: KVSEL_BF16 only */
} kvsel_qevict_desc;

/* Bytes of scratch kvsel_qevict_step needs (0 on invalid arguments). */
size_t kvsel_qevict_step_workspace(const kvsel_qevict_desc* desc);

/*
 * kvsel_qevict_step -- one routing step.  State buffers persist across steps
 * (caller-owned device memory; zero them before the first step: every window
 * full precision, no backing-store entry, score 0).  For every routed window j:
 *   w_acc[j] += the sum of token_scores over its 64 tokens (fp32, a fixed
 *     reduction order); the prompt's attention initialises the scores;
 *   windows not evicted are ranked by (w_acc desc, j asc): the first n_full
 *     are full precision (0), the next n_quant quantised (1), the rest evicted
 *     (2); eviction is permanent;
 *   full -> quantised: if has_codes[j] == 0 the window's K and V rows are
 *     quantised into slot j of the backing store and has_codes[j] = 1;
 *     otherwise the stored codes are kept as they are (no re-quantisation);
 *   quantised -> full: the window's K and V cache rows are overwritten with
 *     bf16_rne(lo + code*scale) (two fp32 roundings, no FMA).
 * Code rule per (window, channel) group of 64 values, K and V separately:
 *   lo = min, scale = (max - lo) / (2^bits - 1) in fp32, code =
 *   clip(rint((x - lo) / scale), 0, 2^bits - 1) (0 when scale == 0); channel c
 *   at bit offset bits*(c mod (8/bits)) of byte c / (8/bits).
 *
 *   token_scores [Bt,Hkv,seq_len] float32, device: this step's attention mass
 *   w_acc        [Bt,Hkv,max_windows] float32 in/out
 *   tier         [Bt,Hkv,max_windows] int8 in/out
 *   has_codes    [Bt,Hkv,max_windows] uint8 in/out
 *   k, v         [Bt,Hkv,capacity,D] bf16 in/out (promotions write rows)
 *   k_codes, v_codes [Bt,Hkv,max_windows,64,D*bits/8] uint8 in/out
 *   k_meta, v_meta   [Bt,Hkv,max_windows,D,2] float32 (lo, scale) in/out
 * Slots j >= nW are not touched.  Errors: KVSEL_ERR_ARG for a bad shape or
 * pointer, nW > max_windows, or negative capacities; KVSEL_ERR_UNSUPPORTED
 * for win != 64, bits not 2 or 4, D not 64/128, a dtype other than bf16, or
 * max_windows > 4096.  Overlapping calls on the same state race.
 */
kvsel_status kvsel_qevict_step(const kvsel_qevict_desc* desc, const float* token_scores,
                               float* w_acc, int8_t* tier, uint8_t* has_codes, void* k, void* v,
                               uint8_t* k_codes, uint8_t* v_codes, float* k_meta, float* v_meta,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_score_static -- kvsel_score for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, outputs and errors, with the
 * scratch taken from a static device array of KVSEL_STATIC_SCRATCH_BYTES
 * inside the library instead of a caller workspace.  No allocation of any
 * kind happens in the call.  Each GPU holds its own copy of the array from
 * the first call on it until the process ends; every call on one GPU shares
 * it, so calls that overlap on one GPU (different streams or threads) race,
 * while calls on one stream are ordered.  A problem whose
 * kvsel_score_workspace(desc) exceeds KVSEL_STATIC_SCRATCH_BYTES returns
 * KVSEL_ERR_WORKSPACE before any device call; KVSEL_ERR_DEVICE if the
 * array's device address cannot be obtained.
 */
#define KVSEL_STATIC_SCRATCH_BYTES (32u << 20)
kvsel_status kvsel_score_static(const kvsel_desc* desc, const void* q_obs, const void* k,
                                float* raw_scores, float* pooled, int32_t pool_kernel,
                                void* stream);

/*
 * Kernel timing for benchmarks (not needed for normal use).
 *
 * kvsel_timing_start(prefix): from now on, every launch of a library kernel
 *   whose name starts with `prefix` ("*" = every kernel) carries a start and
 *   a stop HIP event that its dispatch stamps with the kernel's begin and end
 *   (hipExtLaunchKernel).  NULL or "" stops recording.  Kernel names are those a profiler shows without
 *   template arguments (e.g. "score_pass1_32", "sel_hist", "compact_kernel").
 * kvsel_timing_read: waits for every recorded pair, and writes per kernel
 *   name (in first-launch order, at most max_kernels of them) the name into
 *   names + i*name_bytes (NUL-terminated, truncated), the summed duration in
 *   milliseconds into total_ms[i] and the launch count into launches[i];
 *   the recorded pairs are then released.  Returns the number of distinct
 *   kernel names, -1 on bad arguments, -2 when an event could not be read.
 * Process-wide state behind a mutex; meant for one benchmarking thread.
 */
kvsel_status kvsel_timing_start(const char* kernel_prefix);
int32_t kvsel_timing_read(char* names, int32_t name_bytes, double* total_ms, int32_t* launches,
                          int32_t max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
