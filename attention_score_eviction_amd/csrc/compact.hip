// Retained-row gather (kvsel_compact) for gfx950.
//
// TideKV ("Delayed KV Eviction via Layer-Wise Chunked Prefill ..."),
// Algorithm 2, GATHER(K, V, R): the kept K and V rows are copied, bit for
// bit, into a compact per-KV-head cache.  Each row (D elements, 128-512 B)
// is moved as 16-byte vectors by consecutive lanes, so every wave issues
// fully coalesced 16 B/lane loads and stores.
#include "common.h"

namespace kvsel {
namespace {

// One 16-byte vector of K and one of V per thread: a workgroup moves
// 256 / vpr whole rows, so every thread has a single index -> row load chain
// and all of a workgroup's loads are in flight together.
__global__ void __launch_bounds__(256) compact_kernel(const u32x4_t* __restrict__ k,
                                                      const u32x4_t* __restrict__ v,
                                                      const int32_t* __restrict__ idx,
                                                      u32x4_t* __restrict__ ko,
                                                      u32x4_t* __restrict__ vo, int S,
                                                      int n_keep, int vpr) {
  const int head = blockIdx.y;
  const int rpb = 256 / vpr;
  const int r = blockIdx.x * rpb + threadIdx.x / vpr;
  const int c = threadIdx.x - (threadIdx.x / vpr) * vpr;
  if (r >= n_keep || threadIdx.x >= rpb * vpr) return;
  const int src = idx[(size_t)head * n_keep + r];
  const bool ok = src >= 0 && src < S;
  const size_t so = ((size_t)head * S + (ok ? src : 0)) * vpr + c;
  const size_t dsto = ((size_t)head * n_keep + r) * vpr + c;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const u32x4_t kx = ok ? k[so] : zero;
  if (v) {
    const u32x4_t vx = ok ? v[so] : zero;
    ko[dsto] = kx;
    vo[dsto] = vx;
  } else {
    ko[dsto] = kx;
  }
}

// Flattened head-adaptive cache (TideKV Section 4.1): one row list per
// sequence, head h owning rows [head_off[h], head_off[h+1]).  Rows are moved
// as in compact_kernel (one 16-byte vector of K and one of V per thread); a
// thread's index load is issued before the sequence's offsets are staged in
// LDS, and its head is found there by binary search (in global memory for
// more than kFlatLdsHeads heads), so each thread waits on two loads in a row
// as in the per-head gather.
constexpr int kFlatLdsHeads = 1023;

__device__ __forceinline__ int last_head_at_or_before(const int32_t* off, int hkv, int r) {
  int lo = 0, hi = hkv - 1;   // last head whose first row is <= r (clamped)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256) compact_flat_kernel(const u32x4_t* __restrict__ k,
                                                           const u32x4_t* __restrict__ v,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ head_off,
                                                           u32x4_t* __restrict__ ko,
                                                           u32x4_t* __restrict__ vo, int S,
                                                           int hkv, int n_keep, int vpr) {
  __shared__ int32_t off_s[kFlatLdsHeads + 1];
  const int b = blockIdx.y;
  const int rpb = 256 / vpr;
  const int r = blockIdx.x * rpb + threadIdx.x / vpr;
  const int c = threadIdx.x - (threadIdx.x / vpr) * vpr;
  const bool live = r < n_keep && threadIdx.x < rpb * vpr;
  const int src = live ? idx[(size_t)b * n_keep + r] : -1;
  const int32_t* off = head_off + (size_t)b * (hkv + 1);
  const bool in_lds = hkv <= kFlatLdsHeads;
  if (in_lds)
    for (int i = threadIdx.x; i <= hkv; i += 256) off_s[i] = off[i];
  __syncthreads();
  if (!live) return;
  const int h = last_head_at_or_before(in_lds ? off_s : off, hkv, r);
  const bool ok = src >= 0 && src < S;
  const size_t so = (((size_t)b * hkv + h) * S + (ok ? src : 0)) * vpr + c;
  const size_t dsto = ((size_t)b * n_keep + r) * vpr + c;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const u32x4_t kx = ok ? k[so] : zero;
  if (v) {
    const u32x4_t vx = ok ? v[so] : zero;
    ko[dsto] = kx;
    vo[dsto] = vx;
  } else {
    ko[dsto] = kx;
  }
}

}  // namespace

kvsel_status launch_compact(const kvsel_desc& d, const void* k, const void* v,
                            const int32_t* idx, int n_keep, void* k_out, void* v_out,
                            hipStream_t stream) {
  if (n_keep == 0) return KVSEL_OK;
  const int e = d.dtype == KVSEL_F32 ? 4 : 2;
  const int vpr = d.head_dim * e / 16;
  const int nheads = d.batch * d.n_kv_heads;
  const int rpb = 256 / vpr;   // vpr <= 32 (D * e <= 512 bytes)
  KVSEL_LAUNCH("compact_kernel", compact_kernel, dim3((n_keep + rpb - 1) / rpb, nheads),
                     dim3(256), 0, stream, (const u32x4_t*)k, (const u32x4_t*)v, idx,
                     (u32x4_t*)k_out, (u32x4_t*)v_out, d.seq_len, n_keep, vpr);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

kvsel_status launch_compact_flat(const kvsel_desc& d, const void* k, const void* v,
                                 const int32_t* idx, const int32_t* head_off, int n_keep,
                                 void* k_out, void* v_out, hipStream_t stream) {
  if (n_keep == 0) return KVSEL_OK;
  const int e = d.dtype == KVSEL_F32 ? 4 : 2;
  const int vpr = d.head_dim * e / 16;
  const int rpb = 256 / vpr;   // vpr <= 32 (D * e <= 512 bytes)
  KVSEL_LAUNCH("compact_flat_kernel", compact_flat_kernel,
               dim3((n_keep + rpb - 1) / rpb, d.batch), dim3(256), 0, stream,
               (const u32x4_t*)k, (const u32x4_t*)v, idx, head_off, (u32x4_t*)k_out,
               (u32x4_t*)v_out, d.seq_len, d.n_kv_heads, n_keep, vpr);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
