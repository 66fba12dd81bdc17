// Exact top-B selection with the mandatory set (kvsel_select) for gfx950.
//
// TideKV ("Delayed KV Eviction via Layer-Wise Chunked Prefill ..."),
// Section 4.2, Eq. (8): R = Top_k{p_i : i not mandatory} U mandatory.  The
// pages keep the top-k in a streaming heap inside pass 2 (Algorithm 2); here
// the per-key scores are already a compact fp32 vector per KV head (a few
// MiB, resident in the last-level cache), so the k-th largest value is found
// exactly by a three-digit radix select over the fp32 bit patterns
// (11 + 11 + 10 bits; scores are >= 0, so bit order equals value order).
// Ties at the threshold keep the lowest positions.  The retained positions
// are emitted in ascending order with a block-wide prefix count.
//
// One 1024-thread workgroup per (batch, KV head); histograms live in LDS.
#include "common.h"

namespace kvsel {
namespace {

constexpr int kSelThreads = 1024;

// Exclusive prefix sum over the workgroup; *total receives the sum of all.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total,
                                                         uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kSelThreads / 64 ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kSelThreads / 64; off <<= 1) {
      const uint32_t t = __shfl_up(w, off);
      if (lane >= off) w += t;
    }
    if (lane < kSelThreads / 64) wsum[lane] = w;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[wave - 1] : 0u;
  *total = wsum[kSelThreads / 64 - 1];
  __syncthreads();
  return before + incl - v;
}

// Histogram update with wave-level aggregation: scores cluster in a few
// bins, so lanes sharing a bin are counted by one leader lane (up to two
// distinct bins per wave per call) before the remaining lanes add one each.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int leader = __ffsll((long long)act) - 1;
    const uint32_t lb = __shfl(bin, leader);
    const bool same = active && bin == lb;
    const unsigned long long mk = __ballot(same);
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(mk));
    active = active && !same;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

// Each thread takes 16 consecutive scores per batch as four 16-byte loads
// (scalar loads only at the unaligned ends), so a sweep keeps many bytes in
// flight per CU.  Elements outside [lo, hi) come back invalid.
constexpr int kPerThread = 16;
constexpr int kBatch = kSelThreads * kPerThread;

__device__ __forceinline__ uint32_t load16(const uint32_t* row, int p0, int lo, int hi,
                                           uint32_t (&x)[kPerThread]) {
  uint32_t valid = 0u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int p = p0 + 4 * v;
    if (p >= lo && p + 3 < hi) {
      const u32x4_t w = *(const u32x4_t*)(row + p);
      x[4 * v] = w[0];
      x[4 * v + 1] = w[1];
      x[4 * v + 2] = w[2];
      x[4 * v + 3] = w[3];
      valid |= 0xfu << (4 * v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = p + e;
        const bool ok = i >= lo && i < hi;
        x[4 * v + e] = ok ? row[i] : 0u;
        valid |= (uint32_t)ok << (4 * v + e);
      }
    }
  }
  return valid;
}

__global__ void __launch_bounds__(kSelThreads) select_kernel(const float* __restrict__ pooled,
                                                             int32_t* __restrict__ idx, int S,
                                                             int lo, int hi, int budget,
                                                             int n_sink, int W, int n_keep) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t pick[3];
  const int head = blockIdx.x, tid = threadIdx.x;
  const uint32_t* u = (const uint32_t*)pooled + (size_t)head * S;
  int32_t* out = idx + (size_t)head * n_keep;
  for (int i = tid; i < n_sink; i += kSelThreads) out[i] = i;
  for (int j = tid; j < W; j += kSelThreads) out[n_sink + budget + j] = S - W + j;
  if (budget == 0) return;
  // First batch start: at or below lo, on a 16-byte boundary of the buffer.
  const int ofs = (int)(((size_t)head * S) & 3u);
  const int base0 = lo - ((lo + ofs) & 3);

  // Radix select: digit r covers bits [shift, shift+nbits).
  uint32_t prefix = 0u, pmask = 0u, rem = (uint32_t)budget;
  for (int r = 0; r < 3; ++r) {
    const int shift = r == 0 ? 21 : (r == 1 ? 10 : 0);
    const int nb = r == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int base = base0; base < hi; base += kBatch) {
      uint32_t x[kPerThread];
      const uint32_t valid = load16(u, base + tid * kPerThread, lo, hi, x);
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        hist_add(hist, (x[e] >> shift) & (uint32_t)(nb - 1),
                 ((valid >> e) & 1u) && (x[e] & pmask) == prefix);
    }
    __syncthreads();
    // Thread t owns bins nb-1-2t and nb-2-2t (descending value order).
    const int bA = nb - 1 - 2 * tid, bB = bA - 1;
    uint32_t cA = 0u, cB = 0u;
    if (bB >= 0) {
      cA = hist[bA];
      cB = hist[bB];
    }
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(cA + cB, &tot, wsum);
    if (bB >= 0) {
      if (above < rem && rem <= above + cA) {
        pick[0] = (uint32_t)bA;
        pick[1] = above;
        pick[2] = cA;
      } else if (above + cA < rem && rem <= above + cA + cB) {
        pick[0] = (uint32_t)bB;
        pick[1] = above + cA;
        pick[2] = cB;
      }
    }
    __syncthreads();
    const uint32_t digit = pick[0];
    rem -= pick[1];
    prefix |= digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    const bool whole_bin = rem == pick[2];
    __syncthreads();
    // The whole boundary bin is kept: no need to resolve the lower bits.
    if (whole_bin) break;
  }
  // Kept: (x & pmask) > prefix, and the first `rem` elements (by position)
  // with (x & pmask) == prefix.  After three rounds pmask covers every bit
  // and prefix is the exact bit pattern of the budget-th largest score.
  const uint32_t need_eq = rem;
  uint32_t cgt = 0u, ceq = 0u;
  for (int base = base0; base < hi; base += kBatch) {
    const int i0 = base + tid * kPerThread;
    uint32_t x[kPerThread];
    const uint32_t valid = load16(u, i0, lo, hi, x);
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const uint32_t km = x[e] & pmask;
      const bool ok = (valid >> e) & 1u;
      gt |= (uint32_t)(ok && km > prefix) << e;
      eq |= (uint32_t)(ok && km == prefix) << e;
    }
    const uint32_t ngt = __popc(gt), neq = __popc(eq);
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((ngt << 16) | neq, &tot, wsum);
    uint32_t gtb = cgt + (ex >> 16), eqb = ceq + (ex & 0xffffu);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      // slot < budget always holds for finite non-negative scores; the
      // guard keeps malformed input from writing outside this row.
      if ((gt >> e) & 1u) {
        const uint32_t slot = gtb + min(eqb, need_eq);
        if (slot < (uint32_t)budget) out[n_sink + slot] = i0 + e;
        ++gtb;
      } else if ((eq >> e) & 1u) {
        const uint32_t slot = gtb + eqb;
        if (eqb < need_eq && slot < (uint32_t)budget) out[n_sink + slot] = i0 + e;
        ++eqb;
      }
    }
    cgt += tot >> 16;
    ceq += tot & 0xffffu;
    if (cgt + min(ceq, need_eq) >= (uint32_t)budget && ceq >= need_eq) break;
  }
}

}  // namespace

kvsel_status launch_select(const kvsel_desc& d, const float* pooled, int budget, int32_t* idx,
                           hipStream_t stream) {
  const int nheads = d.batch * d.n_kv_heads;
  const int n_keep = budget + d.n_sink + d.obs_window;
  hipLaunchKernelGGL(select_kernel, dim3(nheads), dim3(kSelThreads), 0, stream, pooled, idx,
                     d.seq_len, d.n_sink, d.seq_len - d.obs_window, budget, d.n_sink,
                     d.obs_window, n_keep);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
