// Internal declarations shared by the kvsel HIP sources (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Optional per-kernel timing (kvsel_timing_start / kvsel_timing_read).  Off by
// default; while a name prefix is set, every launch of a kernel whose name
// starts with it goes through hipExtLaunchKernelGGL with a start and a stop
// event, which the dispatch itself stamps with the kernel's begin and end.
// ---------------------------------------------------------------------------
bool timing_wanted(const char* kernel_name);
bool timing_events(hipEvent_t* start, hipEvent_t* stop);
void timing_record(const char* kernel_name, hipEvent_t start, hipEvent_t stop);

#define KVSEL_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                         \
  do {                                                                                    \
    hipEvent_t kvsel_e0_ = nullptr, kvsel_e1_ = nullptr;                                  \
    if (::kvsel::timing_wanted(NAME) && ::kvsel::timing_events(&kvsel_e0_, &kvsel_e1_)) { \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, kvsel_e0_, kvsel_e1_, 0,  \
                            __VA_ARGS__);                                                 \
      ::kvsel::timing_record(NAME, kvsel_e0_, kvsel_e1_);                                 \
    } else {                                                                              \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                \
    }                                                                                     \
  } while (0)

// Sort key for (value desc, index asc) as one ascending 64-bit integer: the
// value's bits mapped to an order-preserving unsigned form, complemented for
// descending order, above the index.  -0.0 is folded into +0.0 so equal
// values tie; -inf sorts after every finite value; ~0 (padding) after all.
__device__ __forceinline__ uint64_t desc_key(float x, int idx) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in x
  return ((uint64_t)(~ord) << 32) | (uint32_t)idx;
}

// Ascending bitonic sort of key[0, n2) in LDS (n2 a power of two) by a
// workgroup of NT threads.  Every thread of the block must call.
template <int NT>
__device__ __forceinline__ void block_bitonic_sort(uint64_t* key, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = key[i], y = key[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Up to kWaveSortN keys are sorted by one wave in registers, 8 keys per lane
// (element lane*8 + r in x[r]), with no workgroup barrier: the same ascending
// bitonic network, its exchanges at distance j < 8 inside a lane and at
// j >= 8 between lanes lane and lane ^ (j / 8).
constexpr int kWaveSortN = 512;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void wave_bitonic_sort512(uint64_t (&x)[8], int lane) {
#pragma unroll
  for (int k = 2; k <= kWaveSortN; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 8) {
        const bool lower = (lane & (j >> 3)) == 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bool asc = ((lane * 8 + r) & k) == 0;
          const uint64_t y = shfl_xor_u64(x[r], j >> 3);
          // the lower index of the pair keeps the minimum when ascending
          x[r] = (asc == lower) ? (x[r] < y ? x[r] : y) : (x[r] < y ? y : x[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if ((r ^ j) > r) {
            const bool asc = ((lane * 8 + r) & k) == 0;
            const uint64_t a = x[r], b = x[r ^ j];
            const bool sw = (a > b) == asc;
            x[r] = sw ? b : a;
            x[r ^ j] = sw ? a : b;
          }
        }
      }
    }
  }
}

// Ascending sort of key[0, n2) in LDS (n2 a power of two; entries past the
// data hold ~0): by the first wave in registers when n2 <= kWaveSortN, else
// by the whole workgroup of NT threads.  Every thread of the block must
// call; the sorted keys are visible to all threads on return.
template <int NT>
__device__ __forceinline__ void sort_keys(uint64_t* key, int n2) {
  if (n2 <= kWaveSortN) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
      uint64_t x[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int e = lane * 8 + r;
        x[r] = e < n2 ? key[e] : ~0ull;
      }
      wave_bitonic_sort512(x, lane);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int e = lane * 8 + r;
        if (e < n2) key[e] = x[r];
      }
    }
    __syncthreads();
    return;
  }
  block_bitonic_sort<NT>(key, n2);
}

// ---------------------------------------------------------------------------
// Score launch plan.  Keys of one (batch, KV head) are split into chunks of
// `chunk` keys (a multiple of the per-step key count); query rows of the head
// group (G*W of them) are split into groups of at most `qcap` rows.  One
// workgroup handles one (chunk, head, row group).  The result does not depend
// on this split beyond fp32 rounding of the per-chunk statistics.
// ---------------------------------------------------------------------------
struct ScorePlan {
  int nheads;     // Bt * Hkv
  int G;          // query heads per KV head
  int GW;         // query rows per KV head (G * W)
  int GWr;        // GW rounded up to 16
  int maxqt;      // 16-row query tiles per workgroup (template choice)
  int nwaves;     // waves per workgroup
  bool mfma32;    // bf16: 32-row query tiles on 32x32x16 matrix products (maxqt counts them)
  int qcap;       // rows per group = 16 * maxqt
  int ngroups;    // ceil(GW / qcap)
  int chunk;      // keys per workgroup
  int nchunk;     // ceil(S / chunk)
  int fold_tl;    // >= 0: no combine kernel; pass 2 merges the statistics
                  // with 2^fold_tl partial merges per row (few rows and chunks)
  bool keys_lds;  // one launch with the head's keys in LDS (no causal mask,
                  // at most 512 keys, many query rows)
  size_t off_part, off_lse, off_raw, off_grp, total;   // workspace layout (bytes)
};

bool plan_score(const kvsel_desc& d, ScorePlan* p);

struct ScoreArgs {
  const void* q;       // [Bt,Hq,W,D]
  const void* k;       // [Bt,Hkv,S,D]
  float2* part;        // [nheads][GWr][nchunk] (max, sum) in log2 units
  float* lse;          // [nheads][GWr] row log2-sum-exp
  float* s_out;        // [ngroups][nheads][S] (ngroups == 1: the raw scores)
  int Hq, Hkv, G, W, S, GW, GWr, qcap, chunk, nchunk, causal;
  int kstride;         // key rows between consecutive KV heads in k (>= S)
  float c;             // scale * log2(e)
  uint32_t* zero;      // cleared by the combine kernel, or by pass 1 when
  long zero_words;     // pass 2 merges the statistics itself (may be null)
  int fold_tl;         // >= 0: pass 2 merges each row's chunk statistics
                       // itself, in the combine kernel's order with
                       // 2^fold_tl partial merges per row; -1: it reads lse
};

// kstride: key rows per KV head in k (the head's first seq_len rows are
// scored); pooled may be null (no max-pool launched) for callers that only
// need the raw scores.
// zero / zero_words: a buffer the score launch clears on the way (in the
// row-statistics combine, or in pass 1 when there is none), for a select
// that follows on the stream.
kvsel_status launch_score(const kvsel_desc& d, const ScorePlan& p, const void* q, const void* k,
                          float* raw, float* pooled, int pool_kernel, char* ws,
                          hipStream_t stream, int kstride, uint32_t* zero = nullptr,
                          size_t zero_words = 0);
// Streaming top-k (TideKV Algorithm 2's heap in pass 2): per (sequence, KV
// head) row, a list of M candidates (each chunk's top-`budget` pooled scores
// in ascending position order, chunk after chunk) instead of a score vector.
struct StreamArgs {
  float* cval;     // [nheads][M] candidate scores
  int32_t* cpos;   // [nheads][M] their positions
  int lo, hi;      // candidate range [n_sink, S - W)
  int budget, ph, M;
};
// False when the problem does not fit the streaming pass (bf16 prompts of
// 4096 keys or more with one query group per KV head, chunks <= 16384 keys).
bool plan_score_stream(const kvsel_desc& d, ScorePlan* p);
int stream_list_len(const ScorePlan& p, int lo, int hi, int budget);
kvsel_status launch_score_stream(const kvsel_desc& d, const ScorePlan& p, const void* q,
                                 const void* k, const StreamArgs& sa, char* ws,
                                 hipStream_t stream);
kvsel_status launch_stream_finish(const int32_t* sel, const int32_t* cpos, int32_t* idx,
                                  int rows, int M, int budget, int n_sink, int W, int S,
                                  hipStream_t stream);

// Selection groups: hg consecutive KV heads of a sequence share one budget
// (hg = 1: per-head budget; hg = n_kv_heads: head-adaptive budget).
constexpr int kMaxGroupSlices = 2048;
struct SelectPlan {
  bool multi;     // sliced multi-workgroup kernels (long rows, head groups)
  int hg;         // KV heads per selection group
  int groups;     // batch * n_kv_heads / hg
  int ns;         // slices of kSlice scores per KV-head row (sliced kernels)
  int nsl;        // slices of 16 scores per KV-head row (single-workgroup kernel)
  size_t off_hist, off_gtc, off_candc, off_offs, off_params, off_cval, off_cidx, total;
};
// False when a head group needs more than kMaxGroupSlices slices.
bool plan_select(const kvsel_desc& d, int budget, int hg, SelectPlan* p);
kvsel_status launch_select(const kvsel_desc& d, const SelectPlan& p, const float* pooled,
                           int budget, int32_t* idx, int32_t* head_off, char* ws,
                           hipStream_t stream);
// Per-head select and gather in one launch for short rows (else the two).
kvsel_status launch_select_compact(const kvsel_desc& d, const SelectPlan& p, const float* pooled,
                                   int budget, int32_t* idx, const void* k, const void* v,
                                   void* k_out, void* v_out, char* ws, hipStream_t stream);
// The fused max filter, select and gather of the layer-end calls (long
// rows; one KV head per group, or a head group with the flattened gather
// and head_off): from the raw scores, with the digit histograms
// select_hists names zeroed earlier on the stream.
bool layer_end_fusable(const kvsel_desc& d, const SelectPlan& p, int budget, int pool_kernel);
uint32_t* select_hists(const SelectPlan& p, char* ws, size_t* words);
kvsel_status launch_layer_end_select(const kvsel_desc& d, const SelectPlan& p, const float* raw,
                                     float* pooled, int pool_kernel, int budget, int32_t* idx,
                                     int32_t* head_off, const void* k, const void* v,
                                     void* k_out, void* v_out, char* ws, hipStream_t stream);
kvsel_status launch_compact(const kvsel_desc& d, const void* k, const void* v,
                            const int32_t* idx, int n_keep, void* k_out, void* v_out,
                            hipStream_t stream);
kvsel_status launch_compact_flat(const kvsel_desc& d, const void* k, const void* v,
                                 const int32_t* idx, const int32_t* head_off, int n_keep,
                                 void* k_out, void* v_out, hipStream_t stream);

bool kara_supported(int n);
kvsel_status launch_kara_select(const float* scores, int32_t* idx, int rows, int n, int buffer,
                                int keep, int gamma, int alpha, hipStream_t stream);

struct TierPlan {
  int nheads, nwin;
  size_t off_slot, total;
};
bool plan_tiers(const kvsel_tier_desc& d, TierPlan* p);
// Repeated recoverable routing: routed windows of the desc's cache, the
// workspace (one action byte per window slot) and the launch.
int qevict_windows(const kvsel_qevict_desc& d);
size_t qevict_workspace(const kvsel_qevict_desc& d);
kvsel_status launch_qevict(const kvsel_qevict_desc& d, const float* scores, float* w_acc,
                           int8_t* tier, uint8_t* has_codes, void* k, void* v, uint8_t* k_codes,
                           uint8_t* v_codes, float* k_meta, float* v_meta, char* ws,
                           hipStream_t stream);
kvsel_status launch_tiers(const kvsel_tier_desc& d, const TierPlan& p, const float* scores,
                          const void* k, const void* v, int8_t* tier, int32_t* rank,
                          void* k_full, void* v_full, uint8_t* k_codes, uint8_t* v_codes,
                          float* k_meta, float* v_meta, const int32_t* promote, int n_promote,
                          void* k_prom, void* v_prom, char* ws, hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace kvsel
