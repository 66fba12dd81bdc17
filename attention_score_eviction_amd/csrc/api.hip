// C ABI of libkvsel: argument validation and launch sequencing.
//
// Every precondition is checked on the host before anything is enqueued, and
// no check calls the HIP runtime, so invalid calls fail the same way on a
// machine without a GPU.  Environment switches help debugging:
// KVSEL_VALIDATE_ONLY=1 returns after the checks without enqueuing anything,
// KVSEL_SYNC=1 waits for the stream after each call and reports a device
// error as KVSEL_ERR_DEVICE, KVSEL_SCORE_COMBINE=1 keeps the separate
// statistics combine launch for every score plan (read in launch_score).
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

using namespace kvsel;

namespace {

constexpr int64_t kMaxSeq = (int64_t)1 << 28;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}

// Runs the launch sequence of a call whose arguments passed every check,
// honouring KVSEL_VALIDATE_ONLY and KVSEL_SYNC.
template <typename F>
kvsel_status enqueue(void* stream, F&& launch) {
  if (env_flag("KVSEL_VALIDATE_ONLY")) return KVSEL_OK;
  kvsel_status st = launch();
  if (st == KVSEL_OK && env_flag("KVSEL_SYNC")) {
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess || hipGetLastError() != hipSuccess)
      st = KVSEL_ERR_DEVICE;
  }
  return st;
}

kvsel_status check_desc(const kvsel_desc* d) {
  if (!d) return KVSEL_ERR_ARG;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return KVSEL_ERR_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return KVSEL_ERR_ARG;
  if (d->head_dim < 1 || d->seq_len < 1 || d->seq_len > kMaxSeq) return KVSEL_ERR_ARG;
  if (d->obs_window < 1 || d->obs_window > d->seq_len) return KVSEL_ERR_ARG;
  if (d->n_sink < 0 || d->n_sink > d->seq_len - d->obs_window) return KVSEL_ERR_ARG;
  if (d->causal != 0 && d->causal != 1) return KVSEL_ERR_ARG;
  if (d->dtype != KVSEL_BF16 && d->dtype != KVSEL_F32) return KVSEL_ERR_ARG;
  if (!(d->scale >= 0.f) || isinf(d->scale)) return KVSEL_ERR_ARG;
  if ((int64_t)d->batch * d->n_kv_heads > 65535) return KVSEL_ERR_ARG;
  if ((int64_t)(d->n_q_heads / d->n_kv_heads) * d->obs_window > (1 << 20)) return KVSEL_ERR_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
  return KVSEL_OK;
}

kvsel_status check_tier_desc(const kvsel_tier_desc* d) {
  if (!d) return KVSEL_ERR_ARG;
  if (d->batch < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->seq_len < 1) return KVSEL_ERR_ARG;
  if ((int64_t)d->batch * d->n_kv_heads > 65535 || d->seq_len > kMaxSeq) return KVSEL_ERR_ARG;
  if (d->win < 1 || d->seq_len % d->win != 0) return KVSEL_ERR_ARG;
  const int nwin = d->seq_len / d->win;
  if (d->n_full < 0 || d->n_quant < 0 || d->n_full + d->n_quant > nwin) return KVSEL_ERR_ARG;
  if (d->dtype != KVSEL_BF16 && d->dtype != KVSEL_F32) return KVSEL_ERR_ARG;
  if (d->dtype != KVSEL_BF16) return KVSEL_ERR_UNSUPPORTED;
  if (d->win != 64 || nwin > 4096) return KVSEL_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
  return KVSEL_OK;
}

kvsel_status check_qevict_desc(const kvsel_qevict_desc* d) {
  if (!d) return KVSEL_ERR_ARG;
  if (d->batch < 1 || d->n_kv_heads < 1 || d->head_dim < 1) return KVSEL_ERR_ARG;
  if ((int64_t)d->batch * d->n_kv_heads > 65535) return KVSEL_ERR_ARG;
  if (d->seq_len < 0 || d->capacity < d->seq_len || d->capacity > kMaxSeq) return KVSEL_ERR_ARG;
  if (d->n_sink < 0 || d->n_recent < 0 || d->n_full < 0 || d->n_quant < 0) return KVSEL_ERR_ARG;
  if (d->max_windows < 1) return KVSEL_ERR_ARG;
  if (d->win != 64 || (d->bits != 2 && d->bits != 4) || d->max_windows > 4096)
    return KVSEL_ERR_UNSUPPORTED;
  if (d->dtype != KVSEL_BF16) return d->dtype == KVSEL_F32 ? KVSEL_ERR_UNSUPPORTED : KVSEL_ERR_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
  if (qevict_windows(*d) > d->max_windows) return KVSEL_ERR_ARG;
  return KVSEL_OK;
}

// Head-adaptive selection: the sequence-wide pick count must be feasible,
// and a sequence's flattened keys h*S + position must fit in 31 bits.
kvsel_status check_adaptive(const kvsel_desc* d, int32_t total_budget) {
  const kvsel_status st = check_desc(d);
  if (st != KVSEL_OK) return st;
  const int64_t ncand = (int64_t)d->seq_len - d->obs_window - d->n_sink;
  if ((int64_t)d->n_kv_heads * d->seq_len >= ((int64_t)1 << 31)) return KVSEL_ERR_UNSUPPORTED;
  if (total_budget < 0 || total_budget > (int64_t)d->n_kv_heads * ncand) return KVSEL_ERR_BUDGET;
  return KVSEL_OK;
}

kvsel_status check_kara_desc(const kvsel_kara_desc* k) {
  if (!k) return KVSEL_ERR_ARG;
  if (k->batch < 1 || k->n_q_heads < 1 || k->n_kv_heads < 1) return KVSEL_ERR_ARG;
  if (k->n_q_heads % k->n_kv_heads != 0) return KVSEL_ERR_ARG;
  if ((int64_t)k->batch * k->n_kv_heads > 65535) return KVSEL_ERR_ARG;
  if (k->window < 2 || k->window > kMaxSeq || k->buffer < 0 || k->buffer >= k->window)
    return KVSEL_ERR_ARG;
  const int n = k->window - k->buffer;
  if (k->keep < 0 || k->keep > n || k->gamma < 1 || k->alpha < 0) return KVSEL_ERR_ARG;
  if (k->dtype != KVSEL_BF16 && k->dtype != KVSEL_F32) return KVSEL_ERR_ARG;
  if (!(k->scale >= 0.f) || isinf(k->scale)) return KVSEL_ERR_ARG;
  if ((int64_t)(k->n_q_heads / k->n_kv_heads) * k->window > (1 << 20)) return KVSEL_ERR_ARG;
  if (k->head_dim != 64 && k->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
  return KVSEL_OK;
}

// Scoring problem of a Kara window: every window token queries the
// compressible keys (the first window - buffer rows of each head), no mask.
kvsel_desc kara_score_desc(const kvsel_kara_desc& k) {
  kvsel_desc d;
  d.batch = k.batch;
  d.n_q_heads = k.n_q_heads;
  d.n_kv_heads = k.n_kv_heads;
  d.head_dim = k.head_dim;
  d.seq_len = k.window - k.buffer;
  d.obs_window = k.window;
  d.n_sink = 0;
  d.causal = 0;
  d.dtype = (kvsel_dtype)k.dtype;
  d.scale = k.scale;
  return d;
}

}  // namespace

extern "C" {

const char* kvsel_status_str(kvsel_status s) {
  switch (s) {
    case KVSEL_OK: return "ok";
    case KVSEL_ERR_ARG: return "invalid argument";
    case KVSEL_ERR_BUDGET: return "infeasible budget";
    case KVSEL_ERR_WORKSPACE: return "workspace too small";
    case KVSEL_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVSEL_ERR_DEVICE: return "device launch error";
  }
  return "unknown status";
}

size_t kvsel_score_workspace(const kvsel_desc* desc) {
  if (check_desc(desc) != KVSEL_OK) return 0;
  ScorePlan p;
  plan_score(*desc, &p);
  return p.total;
}

kvsel_status kvsel_score(const kvsel_desc* desc, const void* q_obs, const void* k,
                         float* raw_scores, float* pooled, int32_t pool_kernel, void* ws,
                         size_t ws_bytes, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (!q_obs || !k || (!pooled && !raw_scores)) return KVSEL_ERR_ARG;
  if (!aligned16(q_obs) || !aligned16(k) || !aligned16(pooled) || !aligned16(raw_scores))
    return KVSEL_ERR_ARG;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 1 + 2 * (1 << 20))
    return KVSEL_ERR_ARG;
  ScorePlan p;
  plan_score(*desc, &p);
  if (ws_bytes < p.total || (p.total > 0 && !ws)) return KVSEL_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_score(*desc, p, q_obs, k, raw_scores, pooled, pool_kernel, (char*)ws,
                        (hipStream_t)stream, desc->seq_len); });
}

size_t kvsel_select_workspace(const kvsel_desc* desc, int32_t budget) {
  if (check_desc(desc) != KVSEL_OK) return 0;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink) return 0;
  SelectPlan p;
  plan_select(*desc, budget, 1, &p);
  return p.total;
}

kvsel_status kvsel_select(const kvsel_desc* desc, const float* pooled, int32_t budget,
                          int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink)
    return KVSEL_ERR_BUDGET;
  if (!pooled || !idx || !aligned16(pooled) || !aligned16(idx)) return KVSEL_ERR_ARG;
  SelectPlan p;
  plan_select(*desc, budget, 1, &p);
  if (ws_bytes < p.total || (p.total > 0 && !ws)) return KVSEL_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_select(*desc, p, pooled, budget, idx, nullptr, (char*)ws, (hipStream_t)stream); });
}

kvsel_status kvsel_select_compact(const kvsel_desc* desc, const float* pooled, int32_t budget,
                                  int32_t* idx, const void* k, const void* v, void* k_out,
                                  void* v_out, void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink)
    return KVSEL_ERR_BUDGET;
  if (!pooled || !idx || !k || !k_out) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  const void* ptrs[] = {pooled, idx, k, v, k_out, v_out};
  for (const void* q : ptrs)
    if (!aligned16(q)) return KVSEL_ERR_ARG;
  SelectPlan p;
  plan_select(*desc, budget, 1, &p);
  if (ws_bytes < p.total || (p.total > 0 && !ws)) return KVSEL_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_select_compact(*desc, p, pooled, budget, idx, k, v, k_out, v_out, (char*)ws,
                                 (hipStream_t)stream); });
}

// Workspace of kvsel_layer_end: the score scratch, then the select scratch,
// then the pooled scores when the caller does not take them.
struct LayerEndWs {
  ScorePlan sp;
  SelectPlan lp;
  size_t off_sel, off_pooled, total;
};

static LayerEndWs layer_end_ws(const kvsel_desc& d, int budget, bool own_pooled) {
  LayerEndWs w;
  plan_score(d, &w.sp);
  plan_select(d, budget, 1, &w.lp);
  w.off_sel = align256(w.sp.total);
  w.off_pooled = align256(w.off_sel + w.lp.total);
  w.total = w.off_pooled +
            (own_pooled ? align256((size_t)d.batch * d.n_kv_heads * d.seq_len * sizeof(float)) : 0);
  return w;
}

size_t kvsel_layer_end_workspace(const kvsel_desc* desc, int32_t budget) {
  if (check_desc(desc) != KVSEL_OK) return 0;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink) return 0;
  return layer_end_ws(*desc, budget, true).total;
}

kvsel_status kvsel_layer_end(const kvsel_desc* desc, const void* q_obs, const void* k,
                             const void* v, int32_t budget, int32_t pool_kernel,
                             float* raw_scores, float* pooled, int32_t* idx, void* k_out,
                             void* v_out, void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink)
    return KVSEL_ERR_BUDGET;
  if (!q_obs || !k || !idx || !k_out) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  const void* ptrs[] = {q_obs, k, v, raw_scores, pooled, idx, k_out, v_out, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return KVSEL_ERR_ARG;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 1 + 2 * (1 << 20))
    return KVSEL_ERR_ARG;
  const LayerEndWs w = layer_end_ws(*desc, budget, pooled == nullptr);
  if (ws_bytes < w.total || !ws) return KVSEL_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  float* pool_buf = pooled ? pooled : (float*)(wsc + w.off_pooled);
  return enqueue(stream, [&] {
    const hipStream_t s = (hipStream_t)stream;
    char* sel_ws = wsc + w.off_sel;
    if (layer_end_fusable(*desc, w.lp, budget, pool_kernel)) {
      // max filter, select and gather fused behind the two score passes
      float* raw = raw_scores ? raw_scores : (float*)(wsc + w.sp.off_raw);
      size_t words = 0;
      uint32_t* h1 = select_hists(w.lp, sel_ws, &words);
      kvsel_status r = launch_score(*desc, w.sp, q_obs, k, raw, nullptr, pool_kernel, wsc, s,
                                    desc->seq_len, h1, words);
      if (r != KVSEL_OK) return r;
      return launch_layer_end_select(*desc, w.lp, raw, pool_buf, pool_kernel, budget, idx,
                                     nullptr, k, v, k_out, v_out, sel_ws, s);
    }
    kvsel_status r = launch_score(*desc, w.sp, q_obs, k, raw_scores, pool_buf, pool_kernel, wsc,
                                  s, desc->seq_len);
    if (r != KVSEL_OK) return r;
    return launch_select_compact(*desc, w.lp, pool_buf, budget, idx, k, v, k_out, v_out, sel_ws,
                                 s);
  });
}

// Head-adaptive layer end: the score scratch, the head-group select scratch,
// then the pooled scores when the caller does not take them.
struct AdaptiveWs {
  ScorePlan sp;
  SelectPlan lp;
  bool ok;
  size_t off_sel, off_pooled, total;
};

static AdaptiveWs adaptive_ws(const kvsel_desc& d, int total_budget, bool own_pooled) {
  AdaptiveWs w;
  plan_score(d, &w.sp);
  w.ok = plan_select(d, total_budget, d.n_kv_heads, &w.lp);
  w.off_sel = align256(w.sp.total);
  w.off_pooled = align256(w.off_sel + (w.ok ? w.lp.total : 0));
  w.total = w.off_pooled +
            (own_pooled ? align256((size_t)d.batch * d.n_kv_heads * d.seq_len * sizeof(float)) : 0);
  return w;
}

size_t kvsel_layer_end_adaptive_workspace(const kvsel_desc* desc, int32_t total_budget) {
  if (check_adaptive(desc, total_budget) != KVSEL_OK) return 0;
  const AdaptiveWs w = adaptive_ws(*desc, (int)total_budget, true);
  return w.ok ? w.total : 0;
}

kvsel_status kvsel_layer_end_adaptive(const kvsel_desc* desc, const void* q_obs, const void* k,
                                      const void* v, int32_t total_budget, int32_t pool_kernel,
                                      float* raw_scores, float* pooled, int32_t* idx,
                                      int32_t* head_off, void* k_out, void* v_out, void* ws,
                                      size_t ws_bytes, void* stream) {
  const kvsel_status st = check_adaptive(desc, total_budget);
  if (st != KVSEL_OK) return st;
  if (!q_obs || !k || !idx || !head_off || !k_out) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  const void* ptrs[] = {q_obs, k, v, raw_scores, pooled, idx, k_out, v_out, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return KVSEL_ERR_ARG;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 1 + 2 * (1 << 20))
    return KVSEL_ERR_ARG;
  const AdaptiveWs w = adaptive_ws(*desc, (int)total_budget, pooled == nullptr);
  if (!w.ok) return KVSEL_ERR_UNSUPPORTED;
  if (ws_bytes < w.total || !ws) return KVSEL_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  float* pool_buf = pooled ? pooled : (float*)(wsc + w.off_pooled);
  const int n_keep = desc->n_kv_heads * (desc->n_sink + desc->obs_window) + total_budget;
  return enqueue(stream, [&] {
    const hipStream_t s = (hipStream_t)stream;
    char* sel_ws = wsc + w.off_sel;
    if (layer_end_fusable(*desc, w.lp, total_budget, pool_kernel)) {
      // max filter with the first histogram, select and gather behind the passes
      float* raw = raw_scores ? raw_scores : (float*)(wsc + w.sp.off_raw);
      size_t words = 0;
      uint32_t* h = select_hists(w.lp, sel_ws, &words);
      kvsel_status r = launch_score(*desc, w.sp, q_obs, k, raw, nullptr, pool_kernel, wsc, s,
                                    desc->seq_len, h, words);
      if (r != KVSEL_OK) return r;
      return launch_layer_end_select(*desc, w.lp, raw, pool_buf, pool_kernel, total_budget, idx,
                                     head_off, k, v, k_out, v_out, sel_ws, s);
    }
    kvsel_status r = launch_score(*desc, w.sp, q_obs, k, raw_scores, pool_buf, pool_kernel, wsc,
                                  s, desc->seq_len);
    if (r != KVSEL_OK) return r;
    r = launch_select(*desc, w.lp, pool_buf, total_budget, idx, head_off, sel_ws, s);
    if (r != KVSEL_OK) return r;
    return launch_compact_flat(*desc, k, v, idx, head_off, n_keep, k_out, v_out, s);
  });
}

// Streaming path (TideKV Algorithm 2's top-k kept during pass 2): scratch
// is the row statistics, the per-row candidate lists, the merge selection
// and its workspace -- no per-key score vector.
struct StreamWs {
  ScorePlan sp;
  kvsel_desc ld;     // the merge: a selection over the rows' candidate lists
  SelectPlan lp;
  int M;
  size_t off_cval, off_cpos, off_sel, off_lws, total;
};

static bool stream_ws(const kvsel_desc& d, int budget, int pool_kernel, StreamWs* w) {
  if (!plan_score_stream(d, &w->sp) || (pool_kernel - 1) / 2 > 64) return false;
  const int lo = d.n_sink, hi = d.seq_len - d.obs_window;
  w->M = stream_list_len(w->sp, lo, hi, budget);
  w->ld = d;
  w->ld.n_q_heads = d.n_kv_heads;
  w->ld.seq_len = w->M > 0 ? w->M : 1;
  w->ld.obs_window = 0;
  w->ld.n_sink = 0;
  plan_select(w->ld, budget, 1, &w->lp);
  const size_t rows = (size_t)d.batch * d.n_kv_heads;
  size_t off = align256(w->sp.off_raw);   // partials and row statistics only
  w->off_cval = off;
  off = align256(off + rows * w->M * sizeof(float));
  w->off_cpos = off;
  off = align256(off + rows * w->M * sizeof(int32_t));
  w->off_sel = off;
  off = align256(off + rows * budget * sizeof(int32_t));
  w->off_lws = off;
  w->total = off + w->lp.total;
  return true;
}

size_t kvsel_layer_end_stream_workspace(const kvsel_desc* desc, int32_t budget,
                                        int32_t pool_kernel) {
  if (check_desc(desc) != KVSEL_OK) return 0;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink) return 0;
  if (pool_kernel < 1 || pool_kernel % 2 == 0) return 0;
  StreamWs w;
  if (!stream_ws(*desc, budget, pool_kernel, &w)) return 0;
  return w.total;
}

kvsel_status kvsel_layer_end_stream(const kvsel_desc* desc, const void* q_obs, const void* k,
                                    const void* v, int32_t budget, int32_t pool_kernel,
                                    int32_t* idx, void* k_out, void* v_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (budget < 0 || budget > desc->seq_len - desc->obs_window - desc->n_sink)
    return KVSEL_ERR_BUDGET;
  if (!q_obs || !k || !idx || !k_out) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  const void* ptrs[] = {q_obs, k, v, idx, k_out, v_out, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return KVSEL_ERR_ARG;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 1 + 2 * (1 << 20))
    return KVSEL_ERR_ARG;
  StreamWs w;
  if (!stream_ws(*desc, budget, pool_kernel, &w)) return KVSEL_ERR_UNSUPPORTED;
  if (ws_bytes < w.total || !ws) return KVSEL_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  return enqueue(stream, [&] {
    const hipStream_t s = (hipStream_t)stream;
    const int rows = desc->batch * desc->n_kv_heads;
    const int32_t* cpos = (const int32_t*)(wsc + w.off_cpos);
    int32_t* sel = (int32_t*)(wsc + w.off_sel);
    if (budget > 0) {
      StreamArgs sa;
      sa.cval = (float*)(wsc + w.off_cval);
      sa.cpos = (int32_t*)(wsc + w.off_cpos);
      sa.lo = desc->n_sink;
      sa.hi = desc->seq_len - desc->obs_window;
      sa.budget = budget;
      sa.ph = (pool_kernel - 1) / 2;
      sa.M = w.M;
      kvsel_status r = launch_score_stream(*desc, w.sp, q_obs, k, sa, wsc, s);
      if (r != KVSEL_OK) return r;
      r = launch_select(w.ld, w.lp, sa.cval, budget, sel, nullptr, wsc + w.off_lws, s);
      if (r != KVSEL_OK) return r;
    }
    kvsel_status r = launch_stream_finish(sel, cpos, idx, rows, w.M, budget, desc->n_sink,
                                          desc->obs_window, desc->seq_len, s);
    if (r != KVSEL_OK) return r;
    return launch_compact(*desc, k, v, idx, desc->n_sink + budget + desc->obs_window, k_out,
                          v_out, s);
  });
}

size_t kvsel_select_adaptive_workspace(const kvsel_desc* desc, int32_t total_budget) {
  if (check_adaptive(desc, total_budget) != KVSEL_OK) return 0;
  SelectPlan p;
  if (!plan_select(*desc, (int)total_budget, desc->n_kv_heads, &p)) return 0;
  return p.total;
}

kvsel_status kvsel_select_adaptive(const kvsel_desc* desc, const float* pooled,
                                   int32_t total_budget, int32_t* idx, int32_t* head_off,
                                   void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_adaptive(desc, total_budget);
  if (st != KVSEL_OK) return st;
  if (!pooled || !idx || !head_off || !aligned16(pooled) || !aligned16(idx)) return KVSEL_ERR_ARG;
  SelectPlan p;
  if (!plan_select(*desc, (int)total_budget, desc->n_kv_heads, &p)) return KVSEL_ERR_UNSUPPORTED;
  if (ws_bytes < p.total || (p.total > 0 && !ws)) return KVSEL_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_select(*desc, p, pooled, (int)total_budget, idx, head_off, (char*)ws,
                         (hipStream_t)stream); });
}

kvsel_status kvsel_compact(const kvsel_desc* desc, const void* k, const void* v,
                           const int32_t* idx, int32_t n_keep, void* k_out, void* v_out,
                           void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (n_keep < 0) return KVSEL_ERR_ARG;
  if (!k || !k_out || (n_keep > 0 && !idx)) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(idx) || !aligned16(k_out) ||
      !aligned16(v_out))
    return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_compact(*desc, k, v, idx, n_keep, k_out, v_out, (hipStream_t)stream); });
}

kvsel_status kvsel_compact_flat(const kvsel_desc* desc, const void* k, const void* v,
                                const int32_t* idx, const int32_t* head_off, int32_t n_keep,
                                void* k_out, void* v_out, void* stream) {
  const kvsel_status st = check_desc(desc);
  if (st != KVSEL_OK) return st;
  if (n_keep < 0 || n_keep > (int64_t)desc->n_kv_heads * desc->seq_len) return KVSEL_ERR_ARG;
  if (!k || !k_out || (n_keep > 0 && (!idx || !head_off))) return KVSEL_ERR_ARG;
  if ((v == nullptr) != (v_out == nullptr)) return KVSEL_ERR_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(idx) || !aligned16(k_out) ||
      !aligned16(v_out))
    return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_compact_flat(*desc, k, v, idx, head_off, (int)n_keep, k_out, v_out,
                               (hipStream_t)stream); });
}

size_t kvsel_kara_score_workspace(const kvsel_kara_desc* kdesc) {
  if (check_kara_desc(kdesc) != KVSEL_OK) return 0;
  const kvsel_desc d = kara_score_desc(*kdesc);
  ScorePlan p;
  plan_score(d, &p);
  return p.total;
}

kvsel_status kvsel_kara_score(const kvsel_kara_desc* kdesc, const void* q_win, const void* k_win,
                              float* scores, void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_kara_desc(kdesc);
  if (st != KVSEL_OK) return st;
  if (!q_win || !k_win || !scores) return KVSEL_ERR_ARG;
  if (!aligned16(q_win) || !aligned16(k_win) || !aligned16(scores)) return KVSEL_ERR_ARG;
  const kvsel_desc d = kara_score_desc(*kdesc);
  ScorePlan p;
  plan_score(d, &p);
  if (ws_bytes < p.total || (p.total > 0 && !ws)) return KVSEL_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVSEL_ERR_ARG;
  return enqueue(stream, [&] {
    return launch_score(d, p, q_win, k_win, scores, nullptr, 1, (char*)ws, (hipStream_t)stream,
                        kdesc->window); });
}

int32_t kvsel_kara_keep(int32_t window, int32_t buffer, int32_t ratio_num, int32_t ratio_den) {
  if (window < 2 || buffer < 0 || buffer >= window) return -1;
  if (ratio_den < 1 || ratio_num < 0 || ratio_num > ratio_den) return -1;
  const int64_t n = (int64_t)window - buffer;
  // ceil(n * num / den) in integers: exact for every rational ratio
  return (int32_t)((n * ratio_num + ratio_den - 1) / ratio_den);
}

kvsel_status kvsel_kara_select(const kvsel_kara_desc* kdesc, const float* scores, int32_t* idx,
                               void* stream) {
  const kvsel_status st = check_kara_desc(kdesc);
  if (st != KVSEL_OK) return st;
  if (!scores || !idx) return KVSEL_ERR_ARG;
  const int n = kdesc->window - kdesc->buffer;
  if (!kara_supported(n)) return KVSEL_ERR_UNSUPPORTED;
  return enqueue(stream, [&] {
    return launch_kara_select(scores, idx, kdesc->batch * kdesc->n_kv_heads, n, kdesc->buffer,
                              kdesc->keep, kdesc->gamma, kdesc->alpha, (hipStream_t)stream); });
}

size_t kvsel_route_tiers_workspace(const kvsel_tier_desc* desc) {
  if (check_tier_desc(desc) != KVSEL_OK) return 0;
  TierPlan p;
  plan_tiers(*desc, &p);
  return p.total;
}

kvsel_status kvsel_route_tiers(const kvsel_tier_desc* desc, const float* token_scores,
                               const void* k, const void* v, int8_t* tier, int32_t* win_rank,
                               void* k_full, void* v_full, uint8_t* k_codes, uint8_t* v_codes,
                               float* k_meta, float* v_meta, const int32_t* promote,
                               int32_t n_promote, void* k_prom, void* v_prom, void* ws,
                               size_t ws_bytes, void* stream) {
  const kvsel_status st = check_tier_desc(desc);
  if (st != KVSEL_OK) return st;
  if (n_promote < 0) return KVSEL_ERR_ARG;
  if (!token_scores || !k || !v || !tier || !win_rank) return KVSEL_ERR_ARG;
  if (desc->n_full > 0 && (!k_full || !v_full)) return KVSEL_ERR_ARG;
  if (desc->n_quant > 0 && (!k_codes || !v_codes || !k_meta || !v_meta)) return KVSEL_ERR_ARG;
  if (n_promote > 0 && (!promote || !k_prom || !v_prom || desc->n_quant == 0)) return KVSEL_ERR_ARG;
  const void* ptrs[] = {token_scores, k, v, tier, win_rank, k_full, v_full, k_codes,
                        v_codes, k_meta, v_meta, promote, k_prom, v_prom, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return KVSEL_ERR_ARG;
  TierPlan p;
  plan_tiers(*desc, &p);
  if (ws_bytes < p.total || !ws) return KVSEL_ERR_WORKSPACE;
  return enqueue(stream, [&] {
    return launch_tiers(*desc, p, token_scores, k, v, tier, win_rank, k_full, v_full, k_codes,
                        v_codes, k_meta, v_meta, promote, n_promote, k_prom, v_prom, (char*)ws,
                        (hipStream_t)stream); });
}

size_t kvsel_qevict_step_workspace(const kvsel_qevict_desc* desc) {
  if (check_qevict_desc(desc) != KVSEL_OK) return 0;
  return qevict_workspace(*desc);
}

kvsel_status kvsel_qevict_step(const kvsel_qevict_desc* desc, const float* token_scores,
                               float* w_acc, int8_t* tier, uint8_t* has_codes, void* k, void* v,
                               uint8_t* k_codes, uint8_t* v_codes, float* k_meta, float* v_meta,
                               void* ws, size_t ws_bytes, void* stream) {
  const kvsel_status st = check_qevict_desc(desc);
  if (st != KVSEL_OK) return st;
  const void* ptrs[] = {token_scores, w_acc, tier, has_codes, k, v, k_codes, v_codes, k_meta,
                        v_meta, ws};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return KVSEL_ERR_ARG;
  if (ws_bytes < qevict_workspace(*desc)) return KVSEL_ERR_WORKSPACE;
  return enqueue(stream, [&] {
    return launch_qevict(*desc, token_scores, w_acc, tier, has_codes, k, v, k_codes, v_codes,
                         k_meta, v_meta, (char*)ws, (hipStream_t)stream); });
}

}  // extern "C"
