// Workgroup scan, histogram and digit-search helpers of the radix selects
// (gfx950, wave64).  Included by the sources that select inside a workgroup.
#pragma once

#include "common.h"

namespace kvsel {
namespace {

// Inclusive prefix sum across the 64 lanes of a wave: DPP row shifts build
// the sums inside each row of 16 lanes, two row broadcasts carry them across
// rows (no LDS round trips).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over a workgroup of NT threads; *total receives the
// sum of all.  wsum must hold NT/64 entries.  Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total,
                                                         uint32_t* wsum) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
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
  __syncthreads();   // wsum may be reused after this
  return before + incl - v;
}

// Exclusive prefix sum of b over a workgroup of NT threads, and the totals
// of a and of b over all threads, in one pass: two scans per wave, one exchange through
// wsum2 (2*NT/64 entries), two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_pair(uint32_t a, uint32_t b, uint32_t* a_total,
                                                   uint32_t* b_total, uint32_t* wsum2) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    wsum2[wave] = ia;
    wsum2[NWV + wave] = ib;
  }
  __syncthreads();
  uint32_t ta = 0u, tb = 0u, before = 0u;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    ta += wsum2[w];
    tb += wsum2[NWV + w];
    before += w < wave ? wsum2[NWV + w] : 0u;
  }
  *a_total = ta;
  *b_total = tb;
  __syncthreads();
  return before + ib - b;
}

// Histogram update: one LDS atomic per counted score.  (Aggregating equal
// bins across a wave first costs more in cross-lane latency than the atomic
// conflicts it saves, at every row length measured.)
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  if (active) atomicAdd(&hist[bin], 1u);
}

// Histogram update for a thread's kPerThread consecutive scores: runs of
// equal bins (common, since max-pooling repeats a local maximum over its
// neighbours) are counted in registers and added with one atomic per run,
// which cuts same-address conflicts on the crowded bins.
template <int N>
__device__ __forceinline__ void hist_add_runs(uint32_t* hist, const uint32_t (&bin)[N],
                                              uint32_t active) {
  uint32_t cur = bin[0], cnt = active & 1u;
#pragma unroll
  for (int e = 1; e < N; ++e) {
    const bool a = (active >> e) & 1u;
    if (a && bin[e] == cur) {
      ++cnt;
    } else {
      if (cnt) atomicAdd(&hist[cur], cnt);
      cur = bin[e];
      cnt = a ? 1u : 0u;
    }
  }
  if (cnt) atomicAdd(&hist[cur], cnt);
}

// Among the NB bins of `hist` (16-byte aligned), read in descending value
// order, find the bin holding the rem-th largest counted element (rem >= 1
// and at most the total count).  pick[0] = that bin, pick[1] = count strictly
// above it, pick[2] = its own count.  One wave, two levels: each lane sums
// NB/64 consecutive bins and a wave scan finds the lane whose range holds
// the rank; then the wave reads that lane's bins, one per lane, highest
// first, and a second scan finds the bin.  (Keeping a lane's bins in
// registers and walking them serially costs ~100 VGPRs in the kernels that
// inline this.)
template <int NB>
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, uint32_t rem,
                                                uint32_t* pick) {
  constexpr int PER = NB / 64;
  static_assert(PER <= 64 && PER % 4 == 0, "bins per lane");
  const int lane = threadIdx.x & 63;
  uint32_t local = 0u;
  {
    const int b0 = NB - (lane + 1) * PER;
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const u32x4_t w = *(const u32x4_t*)(hist + b0 + j);
      local += (w[0] + w[1]) + (w[2] + w[3]);
    }
  }
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t excl = incl - local;
  const unsigned long long hit = __ballot(excl < rem && rem <= incl);
  if (hit == 0ull) return;
  const int L = __ffsll((long long)hit) - 1;
  const uint32_t run = __builtin_amdgcn_readlane(excl, L);
  const int bin = NB - L * PER - 1 - lane;   // lane 0: lane L's highest bin
  const uint32_t c = lane < PER ? hist[bin] : 0u;
  const uint32_t i2 = wave_incl_scan(c);
  if (lane < PER && run + (i2 - c) < rem && rem <= run + i2) {
    pick[0] = (uint32_t)bin;
    pick[1] = run + (i2 - c);
    pick[2] = c;
  }
}

// wave_find_digit by the first wave, then a barrier so every thread can
// read pick.  Every thread of the block must call.
template <int NB>
__device__ __forceinline__ void block_find_digit(const uint32_t* hist, uint32_t rem,
                                                 uint32_t* pick) {
  if (threadIdx.x < 64) wave_find_digit<NB>(hist, rem, pick);
  __syncthreads();
}

}  // namespace
}  // namespace kvsel
