// Token2Chunk selection over a decode window (kvsel_kara_select) for gfx950.
//
// Kara ("Kara: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
// Compression"), Section 3: the compressible part of the window (its first n
// positions; the buffer U after it is always kept) keeps
//   I  = the `keep` highest importance scores A (Eq. 5),
//   plus the interiors of the floor(alpha / gamma) best chunks between
//   consecutive members of I, a chunk scoring (A[I[k]] + A[I[k+1]]) times
//   its interior length and qualifying only when I[k+1] - I[k] <= gamma
//   (Eqs. 6-8),
//   plus, while fewer than alpha positions were added, the best remaining
//   positions by A (the fill-up rule after Eq. 8).
// Ties go to the lower position (I, fill-up) and to the lower chunk (Eq. 7).
//
// A window holds a few hundred positions, so one 256-thread workgroup takes
// one (sequence, KV head) row entirely in LDS and ranks by counting: every
// position (chunk) counts the ones ordered before it, with broadcast LDS
// reads.  Ascending order for I and for the output comes from block scans.
#include "common.h"

namespace kvsel {
namespace {

constexpr int kKaraThreads = 256;
constexpr int kKaraMax = 2048;   // longest compressible region per row

__device__ __forceinline__ uint32_t kara_wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix over the workgroup; *total gets the sum.  Two barriers.
__device__ __forceinline__ uint32_t kara_block_scan(uint32_t v, uint32_t* total,
                                                    uint32_t* wsum) {
  constexpr int NWV = kKaraThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = kara_wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const uint32_t sw = wsum[w];
    before += w < wave ? sw : 0u;
    tot += sw;
  }
  *total = tot;
  __syncthreads();
  return before + incl - v;
}

// Position states.
constexpr uint8_t kNone = 0, kTop = 1, kChunk = 2, kFill = 3;

// How many of v[0..n4) are ordered before (x0, j0) and before (x1, j1) by
// (value desc, index asc); with STATE only entries whose state is kNone
// count.  Four entries per broadcast LDS read, both probes per read.
// Padding entries hold -inf (never before a finite value) and a state other
// than kNone.
template <bool STATE>
__device__ __forceinline__ void count_before2(const float* v, const uint8_t* st, int n4, float x0,
                                              int j0, float x1, int j1, int& r0, int& r1) {
  int c0 = 0, c1 = 0;
  for (int i = 0; i < n4; i += 4) {
    const float4 q = *(const float4*)&v[i];
    uint32_t sw = 0u;
    if constexpr (STATE) sw = *(const uint32_t*)&st[i];
    const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = !STATE || ((sw >> (8 * u)) & 0xffu) == kNone;
      const int ii = i + u;
      c0 += (ok && (qv[u] > x0 || (qv[u] == x0 && ii < j0))) ? 1 : 0;
      c1 += (ok && (qv[u] > x1 || (qv[u] == x1 && ii < j1))) ? 1 : 0;
    }
  }
  r0 = c0;
  r1 = c1;
}

__global__ void __launch_bounds__(kKaraThreads) kara_select_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx, int n, int buffer, int keep,
    int gamma, int alpha, int n_out) {
  __shared__ __align__(16) float a[kKaraMax];
  __shared__ __align__(16) float rk[kKaraMax];  // chunk scores, < 0 when a chunk does not qualify
  __shared__ int32_t ilist[kKaraMax];           // I in ascending position order
  __shared__ __align__(16) uint8_t state[kKaraMax];
  __shared__ uint32_t wsum[kKaraThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* s = scores + (size_t)row * n;
  int32_t* out = idx + (size_t)row * (n_out + buffer);
  const int n4 = (n + 3) & ~3;
  for (int j = tid; j < n4; j += kKaraThreads) {
    a[j] = j < n ? s[j] : -INFINITY;
    state[j] = j < n ? kNone : kTop;   // padding never counts as a free position
  }
  __syncthreads();

  // Eq. 5: rank by (score desc, position asc); the first `keep` form I.
  for (int base = 0; base < n; base += 2 * kKaraThreads) {
    const int j0 = base + tid, j1 = j0 + kKaraThreads;
    const float x0 = j0 < n ? a[j0] : 0.f, x1 = j1 < n ? a[j1] : 0.f;
    int r0, r1;
    count_before2<false>(a, state, n4, x0, j0, x1, j1, r0, r1);
    if (j0 < n && r0 < keep) state[j0] = kTop;
    if (j1 < n && r1 < keep) state[j1] = kTop;
  }
  __syncthreads();

  // I in ascending order.
  uint32_t nI = 0u;
  for (int base = 0; base < n; base += kKaraThreads) {
    const int j = base + tid;
    const bool f = j < n && state[j] == kTop;
    uint32_t tot;
    const uint32_t ex = kara_block_scan(f ? 1u : 0u, &tot, wsum);
    if (f) ilist[nI + ex] = j;
    nI += tot;
  }
  __syncthreads();

  // Eq. 6: chunk k spans (I[k], I[k+1]); it qualifies when its end points are
  // at most gamma apart.  Scores in fp32: (A + A) * interior length.
  const int nchunk = nI > 1u ? (int)nI - 1 : 0;
  const int nc4 = (nchunk + 3) & ~3;
  for (int k = tid; k < nc4; k += kKaraThreads) {
    float r = -INFINITY;   // padding and non-qualifying chunks rank after every qualifying one
    if (k < nchunk) {
      const int i0 = ilist[k], i1 = ilist[k + 1];
      const int gap = i1 - i0;
      if (gap <= gamma) r = (a[i0] + a[i1]) * (float)(gap - 1);
    }
    rk[k] = r;
  }
  __syncthreads();

  // Eq. 7: the floor(alpha / gamma) best qualifying chunks (score desc, chunk
  // asc); Eq. 8: their interiors join the retained set.  A non-qualifying
  // chunk (-inf) is never counted before a qualifying (finite) one.
  const int want_chunks = alpha / gamma;
  for (int base = 0; base < nchunk; base += 2 * kKaraThreads) {
    const int k0 = base + tid, k1 = k0 + kKaraThreads;
    const float x0 = k0 < nchunk ? rk[k0] : -INFINITY, x1 = k1 < nchunk ? rk[k1] : -INFINITY;
    int r0, r1;
    count_before2<false>(rk, state, nc4, x0, k0, x1, k1, r0, r1);
    if (k0 < nchunk && x0 > -INFINITY && r0 < want_chunks)
      for (int j = ilist[k0] + 1; j < ilist[k0 + 1]; ++j) state[j] = kChunk;
    if (k1 < nchunk && x1 > -INFINITY && r1 < want_chunks)
      for (int j = ilist[k1] + 1; j < ilist[k1 + 1]; ++j) state[j] = kChunk;
  }
  __syncthreads();

  // Fill-up: while fewer than alpha positions were added, the best remaining
  // positions by score (ties to the lower position).
  uint32_t added;
  {
    uint32_t mine = 0u;
    for (int j = tid; j < n; j += kKaraThreads) mine += state[j] == kChunk;
    kara_block_scan(mine, &added, wsum);
  }
  const int need = alpha - (int)added;
  // Decisions are held in registers until every rank is computed, so the
  // ranking reads a state array nobody writes.
  uint32_t fill = 0u;
  if (need > 0) {
    for (int m = 0, base = 0; base < n; m += 2, base += 2 * kKaraThreads) {
      const int j0 = base + tid, j1 = j0 + kKaraThreads;
      const bool f0 = j0 < n && state[j0] == kNone, f1 = j1 < n && state[j1] == kNone;
      if (!f0 && !f1) continue;
      int r0, r1;
      count_before2<true>(a, state, n4, f0 ? a[j0] : 0.f, j0, f1 ? a[j1] : 0.f, j1, r0, r1);
      if (f0 && r0 < need) fill |= 1u << m;
      if (f1 && r1 < need) fill |= 1u << (m + 1);
    }
  }
  __syncthreads();
  for (int m = 0, j = tid; j < n; ++m, j += kKaraThreads)
    if ((fill >> m) & 1u) state[j] = kFill;
  __syncthreads();

  // Retained positions in ascending order, then the buffer.
  uint32_t w = 0u;
  for (int base = 0; base < n; base += kKaraThreads) {
    const int j = base + tid;
    const bool f = j < n && state[j] != kNone;
    uint32_t tot;
    const uint32_t ex = kara_block_scan(f ? 1u : 0u, &tot, wsum);
    // n_out rows for well-formed scores; guarded regardless.
    if (f && w + ex < (uint32_t)n_out) out[w + ex] = j;
    w += tot;
  }
  for (int t = tid; t < buffer; t += kKaraThreads) out[n_out + t] = n + t;
}

}  // namespace

bool kara_supported(int n) { return n >= 1 && n <= kKaraMax; }

kvsel_status launch_kara_select(const float* scores, int32_t* idx, int rows, int n, int buffer,
                                int keep, int gamma, int alpha, hipStream_t stream) {
  const int n_out = keep + alpha < n ? keep + alpha : n;
  hipLaunchKernelGGL(kara_select_kernel, dim3(rows), dim3(kKaraThreads), 0, stream, scores, idx,
                     n, buffer, keep, gamma, alpha, n_out);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
