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
// one (sequence, KV head) row entirely in LDS.  The positions, and then the
// chunks, are put in (score desc, index asc) order by a bitonic sort of
// 64-bit keys (the order is exact: every key is unique) -- in one wave's
// registers for up to 512 keys; ascending order for I and for the output,
// and the fill-up's count of free positions, come from block scans.
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

__global__ void __launch_bounds__(kKaraThreads) kara_select_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx, int n, int buffer, int keep,
    int gamma, int alpha, int n_out) {
  __shared__ float a[kKaraMax];
  __shared__ float rk[kKaraMax];       // chunk scores, -inf when a chunk does not qualify
  __shared__ int32_t ilist[kKaraMax];  // I in ascending position order
  __shared__ uint8_t state[kKaraMax];
  __shared__ uint64_t key[kKaraMax];   // sorted (score desc, position asc), then chunks
  __shared__ uint32_t wsum[kKaraThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* s = scores + (size_t)row * n;
  int32_t* out = idx + (size_t)row * (n_out + buffer);
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int j = tid; j < n2; j += kKaraThreads) {
    if (j < n) {
      const float x = s[j];
      a[j] = x;
      state[j] = kNone;
      key[j] = desc_key(x, j);
    } else {
      key[j] = ~0ull;   // padding sorts last
    }
  }
  __syncthreads();

  // Eq. 5: the first `keep` positions in (score desc, position asc) order form I.
  sort_keys<kKaraThreads>(key, n2);
  for (int r = tid; r < keep; r += kKaraThreads) state[(uint32_t)key[r]] = kTop;
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

  // Fill-up candidates, decided later: the free positions in sorted order.
  // Their sorted order is read now, before the key array is reused.
  constexpr int kPer = kKaraMax / kKaraThreads;
  uint32_t fpos[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int r = m * kKaraThreads + tid;
    fpos[m] = r < n ? (uint32_t)key[r] : 0xffffffffu;
  }
  __syncthreads();

  // Eq. 6: chunk k spans (I[k], I[k+1]); it qualifies when its end points are
  // at most gamma apart.  Scores in fp32: (A + A) * interior length.
  const int nchunk = nI > 1u ? (int)nI - 1 : 0;
  int nc2 = 1;
  while (nc2 < nchunk) nc2 <<= 1;
  for (int k = tid; k < nc2; k += kKaraThreads) {
    if (k < nchunk) {
      const int i0 = ilist[k], i1 = ilist[k + 1];
      const int gap = i1 - i0;
      const float r = gap <= gamma ? (a[i0] + a[i1]) * (float)(gap - 1) : -INFINITY;
      rk[k] = r;
      key[k] = desc_key(r, k);
    } else {
      key[k] = ~0ull;
    }
  }
  __syncthreads();

  // Eq. 7: the floor(alpha / gamma) best qualifying chunks (score desc, chunk
  // asc); Eq. 8: their interiors join the retained set.  A non-qualifying
  // chunk (-inf) sorts after every qualifying one.
  const int want_chunks = alpha / gamma;
  if (nchunk > 0) {
    sort_keys<kKaraThreads>(key, nc2);
    for (int r = tid; r < want_chunks && r < nchunk; r += kKaraThreads) {
      const int k = (int)(uint32_t)key[r];
      if (rk[k] > -INFINITY)
        for (int j = ilist[k] + 1; j < ilist[k + 1]; ++j) state[j] = kChunk;
    }
  }
  __syncthreads();

  // Fill-up: while fewer than alpha positions were added, the best remaining
  // positions by score (ties to the lower position): a prefix count of the
  // free positions in sorted order.
  uint32_t added;
  {
    uint32_t mine = 0u;
    for (int j = tid; j < n; j += kKaraThreads) mine += state[j] == kChunk;
    kara_block_scan(mine, &added, wsum);
  }
  const int need = alpha - (int)added;
  uint32_t fill = 0u;
  if (need > 0) {
    uint32_t seen = 0u;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (m * kKaraThreads >= n) break;
      const bool f = fpos[m] != 0xffffffffu && state[fpos[m]] == kNone;
      uint32_t tot;
      const uint32_t ex = kara_block_scan(f ? 1u : 0u, &tot, wsum);
      if (f && seen + ex < (uint32_t)need) fill |= 1u << m;
      seen += tot;
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kPer; ++m)
    if ((fill >> m) & 1u) state[fpos[m]] = kFill;
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
  // keep + alpha in 64 bits: alpha may be any non-negative int32
  const int n_out = (int64_t)keep + alpha < (int64_t)n ? keep + alpha : n;
  KVSEL_LAUNCH("kara_select_kernel", kara_select_kernel, dim3(rows), dim3(kKaraThreads), 0, stream, scores, idx,
                     n, buffer, keep, gamma, alpha, n_out);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
