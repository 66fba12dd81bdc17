// Observation-window key scoring (kvsel_score) for gfx950.
//
// TideKV ("Delayed KV Eviction via Layer-Wise Chunked Prefill ..."),
// Section 4.2: the logits of Eq. (4) are streamed over key blocks twice.
// Pass 1 finds each query row's running maximum and normaliser (Eqs. 5-6);
// pass 2 recomputes the logits, normalises them (Eq. 7, left) and sums them
// over the window queries and the GQA group (Eq. 7, right, unit weights).
// A 1-D max filter over the candidate positions then smooths the per-key
// scores (Algorithm 2, "pool to p_i").
//
// Kernel design (CDNA4, wave64):
//  * One workgroup = one chunk of keys x one KV head x one group of up to
//    qcap query rows.  The group's query rows are staged once in LDS in MFMA
//    fragment order by direct global->LDS copies (every ds_read_b128 is a
//    contiguous, conflict-free 1 KiB).
//  * Every wave streams its own 64-key blocks straight from HBM into
//    registers (each lane reads the contiguous bytes of one key row that
//    form its MFMA operand fragment), then loops over the query tiles in
//    LDS.  Waves never synchronise inside the key loop.
//  * bf16 prompts of 4096 keys or more use v_mfma_f32_32x32x16_bf16 on
//    32-row query tiles (score_pass1_32 / score_pass2_32); shorter ones and
//    fp32 inputs use the 16x16 forms (score_pass1 / score_pass2).  The
//    operand roles are swapped between the passes so that the dimension each
//    pass reduces over stays inside a lane: pass 1 puts keys on the MFMA rows
//    (each lane keeps running max/sum for one query row), pass 2 puts query
//    rows on the MFMA rows (each lane keeps the running column sum for one
//    key).
//  * Pass 1 leaves per-chunk (max, sum) partials; score_combine merges them
//    per row before pass 2, or, for plans with few rows and chunks, every
//    pass-2 workgroup merges them itself in the same order (no launch).
//  * Unmasked scoring of many query rows over at most 512 keys (a decode
//    window scoring its own keys) runs both passes in one launch per KV head
//    with the head's keys in LDS (score_keys_lds32).
//  * Exponentials are exp2 with scale*log2(e) folded into one FMA per logit.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "common.h"
#include "select_util.h"

namespace kvsel {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int NV>
struct Frag {
  u32x4_t v[NV];
};

// 16-byte vectors per lane for one 16-row x D tile.
template <typename T, int D>
constexpr int nvec() { return D * (int)sizeof(T) / 64; }

// Lane (row r = lane%16, group g = lane/16) holds vectors v = 0..NV-1 covering
// elements [(4v+g)*16/e, +16/e) of its row.  A and B operands use the same
// element-to-k assignment, so the contraction covers every d exactly once.
template <int NV>
__device__ __forceinline__ void load_frag_global(Frag<NV>& f, const char* row_bytes, int g) {
#pragma unroll
  for (int i = 0; i < NV; ++i) f.v[i] = *(const u32x4_t*)(row_bytes + (4 * i + g) * 16);
}

template <typename T, int NV>
__device__ __forceinline__ f32x4_t mma(const Frag<NV>& a, const Frag<NV>& b, f32x4_t c) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v[i]),
                                                  __builtin_bit_cast(bf16x8_t, b.v[i]), c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v[i][e]),
                                                 __uint_as_float(b.v[i][e]), c, 0, 0, 0);
  }
  return c;
}

// Stage query rows [0, nrows) of a group (row-major, D elements each) into LDS
// in fragment order: vector (tile t, v, lane) at index (t*NV + v)*64 + lane.
// Each wave copies whole 1 KiB fragment vectors straight from global memory
// into LDS (global_load_lds_dwordx4), so no registers hold the data and all
// copies are in flight together.  Rows past nrows repeat the last row; their
// results are never used (pass 1 drops their statistics, pass 2 gives them an
// infinite normaliser).
template <typename T, int D, int NT>
__device__ __forceinline__ void stage_queries(u32x4_t* qs, const T* qg, int nrows, int nqt) {
  constexpr int NV = nvec<T, D>();
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  for (int tv = wave; tv < nqt * NV; tv += NW) {
    const int t = tv / NV, v = tv - t * NV;
    const int row = min(t * 16 + (lane & 15), nrows - 1);
    const char* src = (const char*)(qg + (size_t)row * D) + (4 * v + g) * 16;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)(qs + tv * 64),
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

__device__ __forceinline__ void lse_merge(float& m, float& z, float mo, float zo) {
  const float mn = fmaxf(m, mo);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  // one explicit fma, so every caller rounds alike
  z = fmaf(z, __builtin_amdgcn_exp2f(m - mu), zo * __builtin_amdgcn_exp2f(mo - mu));
  m = mn;
}

// The combine kernel's row statistics, computed inside pass 2 for plans
// with few rows and chunks (no combine launch): the workgroup's threads take
// the combine's lanes in its order, tpr = 2^tl adjacent lanes per row, lane
// sub merging chunks sub, sub + tpr, sub + 2 tpr, sub + 3 tpr (the one block
// of four each combine lane takes when nchunk <= 4 tpr, which the plan
// keeps) and the same xor-shuffle tree, so the result is the combine's bit
// for bit, with the loads of adjacent lanes coalesced.  Chunks past the end
// merge (-inf, 0), which leaves (m, z) unchanged (fma(z, 2^0, 0)), so no
// merge needs a branch; their z is the loaded sum times 0 (sums are finite
// and >= 0), so every load is used and stays unconditional.  ls[r] receives
// row r's log2-sum-exp for r < nrows.
constexpr int kFoldMaxTpr = 8;

template <int NT, int ROWS>
struct FoldRows {
  static constexpr int IT = (ROWS * kFoldMaxTpr + NT - 1) / NT;
  float2 pz[IT][4];

  // The loads, issued early (nothing waits for them until merge()).
  __device__ __forceinline__ void load(const float2* __restrict__ part, int nchunk, int tl,
                                       int nrows) {
    const int tpr = 1 << tl, tasks = ROWS << tl, tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int it = min(i * NT + tid, tasks - 1);
      const int row = min(it >> tl, nrows - 1), sub = it & (tpr - 1);
      const float2* p = part + (size_t)row * nchunk;
#pragma unroll
      for (int j = 0; j < 4; ++j) pz[i][j] = p[min(sub + j * tpr, nchunk - 1)];
    }
  }

  __device__ __forceinline__ void merge(int nchunk, int tl, int nrows, float* ls) const {
    const int tpr = 1 << tl, tasks = ROWS << tl, tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      if (i * NT >= tasks) break;   // uniform over the workgroup
      const int it = i * NT + tid;
      const int row = it >> tl, sub = it & (tpr - 1);
      float m = -INFINITY, z = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = it < tasks && row < nrows && sub + j * tpr < nchunk;
        lse_merge(m, z, in ? pz[i][j].x : -INFINITY, pz[i][j].y * (in ? 1.f : 0.f));
      }
      for (int off = tpr >> 1; off >= 1; off >>= 1) {
        const float mo = __shfl_xor(m, off);
        const float zo = __shfl_xor(z, off);
        lse_merge(m, z, mo, zo);
      }
      if (it < tasks && row < nrows && sub == 0) ls[row] = m + log2f(z);
    }
  }
};

// Causal limit of a query row: the last key it may see.
__device__ __forceinline__ int key_limit(const ScoreArgs& a, int qrow) {
  return a.causal ? min(a.S - a.W + (qrow % a.W), a.S - 1) : (a.S - 1);
}

template <int NV>
__device__ __forceinline__ void load_key_block(Frag<NV> (&kf)[4], const char* kh, int kb, int S,
                                               int row_bytes, int l16, int g) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int row = min(kb + kt * 16 + l16, S - 1);
    load_frag_global<NV>(kf[kt], kh + (size_t)row * row_bytes, g);
  }
}

// One 64-key block of pass 1 against all NQT query tiles.  MFMAs of tile
// t+1 are issued before the exp work of tile t.  MASK applies the causal /
// tail mask (only the blocks that reach the window or the end of the keys).
template <typename T, int NV, int NQT, bool MASK>
__device__ __forceinline__ void pass1_block(const int* lims, const Frag<NV> (&kf)[4],
                                            const u32x4_t* qs, float (&m)[NQT],
                                            float (&z)[NQT], int kb, int row0, int lane, int g,
                                            int l16, float c) {
  f32x4_t acc[2][4];
  {
    Frag<NV> qf;
#pragma unroll
    for (int i = 0; i < NV; ++i) qf.v[i] = qs[i * 64 + lane];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      acc[0][kt] = mma<T, NV>(kf[kt], qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    f32x4_t(&cur)[4] = acc[t & 1];
    if (t + 1 < NQT) {
      Frag<NV> qf;
#pragma unroll
      for (int i = 0; i < NV; ++i) qf.v[i] = qs[((t + 1) * NV + i) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        acc[(t + 1) & 1][kt] = mma<T, NV>(kf[kt], qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
    }
    // cur[kt][i]: key kb + kt*16 + 4g + i, query row t*16 + l16
    if constexpr (MASK) {
      const int lim = lims[t * 16 + l16];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + kt * 16 + 4 * g + i > lim) cur[kt][i] = -INFINITY;
    }
    // Maximum of the 16 logits as three-input maxima (v_max3_f32): 8 ops.
    const float a0 = max3f(cur[0][0], cur[0][1], cur[0][2]);
    const float a1 = max3f(cur[0][3], cur[1][0], cur[1][1]);
    const float a2 = max3f(cur[1][2], cur[1][3], cur[2][0]);
    const float a3 = max3f(cur[2][1], cur[2][2], cur[2][3]);
    const float a4 = max3f(cur[3][0], cur[3][1], cur[3][2]);
    const float mx = max3f(max3f(a0, a1, a2), max3f(a3, a4, cur[3][3]), -INFINITY);
    const float mnew = fmaxf(m[t], mx * c);
    const float mu = (mnew == -INFINITY) ? 0.f : mnew;
    // All exponentials first, then the sums: no add waits on a fresh
    // transcendental result.
    float e[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[kt * 4 + i] = __builtin_amdgcn_exp2f(fmaf(cur[kt][i], c, -mu));
    const float sum = (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]))) +
                      (((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15])));
    z[t] = z[t] * __builtin_amdgcn_exp2f(m[t] - mu) + sum;
    m[t] = mnew;
    
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 64-key block of pass 2: as[kt] collects, for key kb + kt*16 + l16, the
// normalised weights of the query rows 4g..4g+3 of every tile.
template <typename T, int NV, int NQT, bool MASK>
__device__ __forceinline__ void pass2_block(const int* lims, const Frag<NV> (&kf)[4],
                                            const u32x4_t* qs, const float* ls,
                                            float (&as)[4], int kb, int row0, int lane, int g,
                                            int l16, float c) {
  f32x4_t acc[2][4];
  {
    Frag<NV> qf;
#pragma unroll
    for (int i = 0; i < NV; ++i) qf.v[i] = qs[i * 64 + lane];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      acc[0][kt] = mma<T, NV>(qf, kf[kt], f32x4_t{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    f32x4_t(&cur)[4] = acc[t & 1];
    if (t + 1 < NQT) {
      Frag<NV> qf;
#pragma unroll
      for (int i = 0; i < NV; ++i) qf.v[i] = qs[((t + 1) * NV + i) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        acc[(t + 1) & 1][kt] = mma<T, NV>(qf, kf[kt], f32x4_t{0.f, 0.f, 0.f, 0.f});
    }
    // cur[kt][i]: query row t*16 + 4g + i, key kb + kt*16 + l16
    const f32x4_t lq = *(const f32x4_t*)&ls[t * 16 + 4 * g];
    if constexpr (MASK) {
      const int4 lim = *(const int4*)&lims[t * 16 + 4 * g];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int key = kb + kt * 16 + l16;
        if (key > lim.x) cur[kt][0] = -INFINITY;
        if (key > lim.y) cur[kt][1] = -INFINITY;
        if (key > lim.z) cur[kt][2] = -INFINITY;
        if (key > lim.w) cur[kt][3] = -INFINITY;
      }
    }
    float e[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[kt * 4 + i] = __builtin_amdgcn_exp2f(fmaf(cur[kt][i], c, -lq[i]));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      as[kt] += (e[kt * 4] + e[kt * 4 + 1]) + (e[kt * 4 + 2] + e[kt * 4 + 3]);
    
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Pass 1: per (chunk, head, row group) partial (max, sum of exp2) per query row.
// NQT = query tiles of 16 rows handled by every wave (rows past the group's
// end are zero and their statistics are dropped).
// ---------------------------------------------------------------------------
template <typename T, int D, int NQT, int NW>
__global__ void __launch_bounds__(NW * 64) score_pass1(ScoreArgs a) {
  constexpr int NV = nvec<T, D>();
  constexpr int NT = NW * 64;
  constexpr int RB = D * (int)sizeof(T);
  __shared__ u32x4_t qs[NQT * NV * 64];
  __shared__ int lims[NQT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int chunk = blockIdx.x, head = blockIdx.y, grp = blockIdx.z;
  const int b = head / a.Hkv, hk = head - b * a.Hkv;
  const int row0 = grp * a.qcap;
  const int nrows = min(a.qcap, a.GW - row0);
  const int S = a.S;
  const float c = a.c;
  const char* kh = (const char*)((const T*)a.k + (size_t)head * a.kstride * D);
  const int k0 = chunk * a.chunk;
  const int kend = min(S, k0 + a.chunk);
  const int mask_from = a.causal ? (S - a.W + 1) : S;

  // Issue this wave's first key block before staging the queries.
  int kb = k0 + wave * 64;
  Frag<NV> kf[4];
  if (kb < kend) load_key_block<NV>(kf, kh, kb, S, RB, l16, g);
  const T* qg = (const T*)a.q + ((size_t)(b * a.Hq + hk * a.G) * a.W + row0) * D;
  stage_queries<T, D, NT>(qs, qg, nrows, NQT);
  for (int r = tid; r < NQT * 16; r += NT) lims[r] = key_limit(a, row0 + r);
  __syncthreads();

  float m[NQT], z[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) { m[t] = -INFINITY; z[t] = 0.f; }

  for (; kb < kend; kb += NW * 64) {
    // Prefetch the next block into registers while this one is consumed.
    Frag<NV> kn[4];
    const bool has_next = kb + NW * 64 < kend;
    if (has_next) load_key_block<NV>(kn, kh, kb + NW * 64, S, RB, l16, g);
    // An opaque zero offset makes the query-fragment reads loop-variant, so
    // they are re-read from LDS every block instead of all being kept live
    // in registers (16 VGPRs per tile).
    int lds_off = 0;
    asm volatile("" : "+v"(lds_off));
    const u32x4_t* qsv = qs + lds_off;
    if (kb + 64 > mask_from)
      pass1_block<T, NV, NQT, true>(lims, kf, qsv, m, z, kb, row0, lane, g, l16, c);
    else
      pass1_block<T, NV, NQT, false>(lims, kf, qsv, m, z, kb, row0, lane, g, l16, c);
    if (has_next) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = kn[kt];
    }
  }

  // Lanes l16, l16+16, l16+32, l16+48 hold partials of the same query row.
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = __shfl_xor(m[t], off);
      const float zo = __shfl_xor(z[t], off);
      lse_merge(m[t], z[t], mo, zo);
    }
  }
  __syncthreads();  // the query tiles are no longer read
  float2* red = (float2*)qs;  // [NW][NQT*16]
  if (g == 0) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) red[wave * NQT * 16 + t * 16 + l16] = make_float2(m[t], z[t]);
  }
  __syncthreads();
  for (int r = tid; r < nrows; r += NT) {
    float mm = -INFINITY, zz = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float2 pz = red[w * NQT * 16 + r];
      lse_merge(mm, zz, pz.x, pz.y);
    }
    // partials laid out [head][row][chunk] so the combine reads them contiguously
    a.part[((size_t)head * a.GWr + row0 + r) * a.nchunk + chunk] = make_float2(mm, zz);
  }
}

// ---------------------------------------------------------------------------
// bf16 passes on v_mfma_f32_32x32x16_bf16.  A 32x32 matrix product keeps the
// matrix core busy twice as long per instruction as the 16x16x32 form and
// overlaps far better with the exponential / sum VALU work of the passes
// (in-wave probe: MFMA stream + softmax VALU 548 cycles vs 705 for the same
// work on 16x16x32; the VALU alone 504).
//  * Query tiles are 32 rows, key tiles 32 keys; a 64-key block is two key
//    tiles.  Lane (r = lane % 32, h = lane / 32) holds, of its tile's row r,
//    the D/2 contiguous elements [h*D/2, (h+1)*D/2): its D bytes are its
//    operand for all D/16 k-steps (step s takes elements h*D/2 + 8s .. +7, the
//    same on both operands, so every d is covered once).
//  * Result element i of lane l is (row 8*(i/4) + 4*h + i%4, column l % 32).
// ---------------------------------------------------------------------------
template <int NV>
__device__ __forceinline__ f32x16_t mma32(const Frag<NV>& a, const Frag<NV>& b, f32x16_t c) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v[i]),
                                                __builtin_bit_cast(bf16x8_t, b.v[i]), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Two 32-key tiles starting at kb (rows past the end repeat the last key).
template <int D>
__device__ __forceinline__ void load_key_block32(Frag<D / 16> (&kf)[2], const char* kh, int kb,
                                                 int S, int lane) {
  constexpr int RB = D * 2;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int row = min(kb + kt * 32 + r, S - 1);
    const char* src = kh + (size_t)row * RB + h * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) kf[kt].v[i] = *(const u32x4_t*)(src + 16 * i);
  }
}

// Query rows [0, nrows) of a group into LDS in fragment order: vector
// (tile t, v, lane) at (t*NV + v)*64 + lane; direct global->LDS copies.
template <int D, int NT>
__device__ __forceinline__ void stage_queries32(u32x4_t* qs, const uint16_t* qg, int nrows,
                                                int nqt) {
  constexpr int NV = D / 16;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int tv = wave; tv < nqt * NV; tv += NW) {
    const int t = tv / NV, v = tv - t * NV;
    const int row = min(t * 32 + (lane & 31), nrows - 1);
    const char* src = (const char*)(qg + (size_t)row * D) + (lane >> 5) * D + 16 * v;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)(qs + tv * 64),
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

__device__ __forceinline__ float max16(const f32x16_t& x) {
  const float a0 = max3f(x[0], x[1], x[2]), a1 = max3f(x[3], x[4], x[5]);
  const float a2 = max3f(x[6], x[7], x[8]), a3 = max3f(x[9], x[10], x[11]);
  const float a4 = max3f(x[12], x[13], x[14]);
  return max3f(max3f(a0, a1, a2), max3f(a3, a4, x[15]), -INFINITY);
}

// Pass 1 on one 64-key block: lane (r, h) keeps the running (max, sum) of
// query row t*32 + r over its 16 keys per key tile.
template <int NV, int NQ, bool MASK>
__device__ __forceinline__ void pass1_block32(const int* lims, const Frag<NV> (&kf)[2],
                                              const u32x4_t* qs, float (&m)[NQ], float (&z)[NQ],
                                              int kb, int lane, float c) {
  const int r = lane & 31, h = lane >> 5;
  f32x16_t acc[2][2];
  {
    Frag<NV> qf;
#pragma unroll
    for (int i = 0; i < NV; ++i) qf.v[i] = qs[i * 64 + lane];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) acc[0][kt] = mma32<NV>(kf[kt], qf, zero16());
  }
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    f32x16_t(&cur)[2] = acc[t & 1];
    if (t + 1 < NQ) {
      Frag<NV> qf;
#pragma unroll
      for (int i = 0; i < NV; ++i) qf.v[i] = qs[((t + 1) * NV + i) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[(t + 1) & 1][kt] = mma32<NV>(kf[kt], qf, zero16());
    }
    // cur[kt][i]: key kb + kt*32 + 8*(i/4) + 4h + i%4, query row t*32 + r
    if constexpr (MASK) {
      const int lim = lims[t * 32 + r];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3) > lim) cur[kt][i] = -INFINITY;
    }
    const float mx = fmaxf(max16(cur[0]), max16(cur[1]));
    const float mnew = fmaxf(m[t], mx * c);
    const float mu = (mnew == -INFINITY) ? 0.f : mnew;
    float e[32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) e[kt * 16 + i] = __builtin_amdgcn_exp2f(fmaf(cur[kt][i], c, -mu));
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) e[i] += e[i + w];
    z[t] = z[t] * __builtin_amdgcn_exp2f(m[t] - mu) + e[0];
    m[t] = mnew;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Pass 2 on one 64-key block: as[kt] collects, for key kb + kt*32 + r, the
// normalised weights of the query rows 8j + 4h + q (j, q < 4) of every tile.
template <int NV, int NQ, bool MASK>
__device__ __forceinline__ void pass2_block32(const int* lims, const Frag<NV> (&kf)[2],
                                              const u32x4_t* qs, const float* ls, float (&as)[2],
                                              int kb, int lane, float c) {
  const int r = lane & 31, h = lane >> 5;
  f32x16_t acc[2][2];
  {
    Frag<NV> qf;
#pragma unroll
    for (int i = 0; i < NV; ++i) qf.v[i] = qs[i * 64 + lane];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) acc[0][kt] = mma32<NV>(qf, kf[kt], zero16());
  }
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    f32x16_t(&cur)[2] = acc[t & 1];
    if (t + 1 < NQ) {
      Frag<NV> qf;
#pragma unroll
      for (int i = 0; i < NV; ++i) qf.v[i] = qs[((t + 1) * NV + i) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[(t + 1) & 1][kt] = mma32<NV>(qf, kf[kt], zero16());
    }
    // cur[kt][i]: query row t*32 + 8*(i/4) + 4h + i%4, key kb + kt*32 + r
    f32x4_t lq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lq[j] = *(const f32x4_t*)&ls[t * 32 + 8 * j + 4 * h];
    if constexpr (MASK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int4 lim = *(const int4*)&lims[t * 32 + 8 * j + 4 * h];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = kb + kt * 32 + r;
          if (key > lim.x) cur[kt][4 * j] = -INFINITY;
          if (key > lim.y) cur[kt][4 * j + 1] = -INFINITY;
          if (key > lim.z) cur[kt][4 * j + 2] = -INFINITY;
          if (key > lim.w) cur[kt][4 * j + 3] = -INFINITY;
        }
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        e[i] = __builtin_amdgcn_exp2f(fmaf(cur[kt][i], c, -lq[i >> 2][i & 3]));
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) e[i] += e[i + w];
      as[kt] += e[0];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Two waves share each SIMD (waves w and w + NW/2 of an 8-wave workgroup).
// The older one wins issue ties and, with equal static shares of key blocks,
// finishes far ahead of the other (measured: 62 against 87 us of a 128K
// pass), which then runs alone.  After each block a wave raises its priority
// while it is behind its partner, so both advance evenly.  Results do not
// depend on it (the block assignment is static).
template <int NW>
__device__ __forceinline__ void pace_partner(int* prog, int wave, int lane, int& nblk) {
  if constexpr (NW == 8) {
    ++nblk;
    if (lane == 0) prog[wave] = nblk;
    const int other = __builtin_amdgcn_readfirstlane(prog[wave ^ (NW / 2)]);
    if (nblk > other) __builtin_amdgcn_s_setprio(0);
    else __builtin_amdgcn_s_setprio(2);
  }
}

template <int D, int NQ, int NW>
__global__ void __launch_bounds__(NW * 64) score_pass1_32(ScoreArgs a) {
  constexpr int NV = D / 16;
  constexpr int NT = NW * 64;
  __shared__ u32x4_t qs[NQ * NV * 64];
  __shared__ int lims[NQ * 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, head = blockIdx.y, grp = blockIdx.z;
  const int b = head / a.Hkv, hk = head - b * a.Hkv;
  const int row0 = grp * a.qcap;
  const int nrows = min(a.qcap, a.GW - row0);
  const int S = a.S;
  const float c = a.c;
  const char* kh = (const char*)((const uint16_t*)a.k + (size_t)head * a.kstride * D);
  const int k0 = chunk * a.chunk;
  const int kend = min(S, k0 + a.chunk);
  const int mask_from = a.causal ? (S - a.W + 1) : S;

  int kb = k0 + wave * 64;
  Frag<NV> kf[2];
  if (kb < kend) load_key_block32<D>(kf, kh, kb, S, lane);
  const uint16_t* qg = (const uint16_t*)a.q + ((size_t)(b * a.Hq + hk * a.G) * a.W + row0) * D;
  stage_queries32<D, NT>(qs, qg, nrows, NQ);
  for (int r = tid; r < NQ * 32; r += NT) lims[r] = key_limit(a, row0 + r);
  if (a.fold_tl >= 0 && a.zero) {
    // no combine launch follows: the select's buffer is cleared here
    const long nthr = (long)gridDim.x * gridDim.y * gridDim.z * NT;
    const long gt = ((long)(blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * NT + tid;
    for (long i = gt; i < a.zero_words; i += nthr) a.zero[i] = 0u;
  }
  __shared__ int prog[NW];
  if (tid < NW) prog[tid] = 0;
  int nblk = 0;
  __syncthreads();

  float m[NQ], z[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) { m[t] = -INFINITY; z[t] = 0.f; }
  for (; kb < kend; kb += NW * 64) {
    int lds_off = 0;
    asm volatile("" : "+v"(lds_off));
    const u32x4_t* qsv = qs + lds_off;
    if (kb + 64 > mask_from)
      pass1_block32<NV, NQ, true>(lims, kf, qsv, m, z, kb, lane, c);
    else
      pass1_block32<NV, NQ, false>(lims, kf, qsv, m, z, kb, lane, c);
    if (kb + NW * 64 < kend) load_key_block32<D>(kf, kh, kb + NW * 64, S, lane);
    pace_partner<NW>(prog, wave, lane, nblk);
  }
  __builtin_amdgcn_s_setprio(0);
  // Lanes r and r + 32 hold partials of the same query row.
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const float mo = __shfl_xor(m[t], 32);
    const float zo = __shfl_xor(z[t], 32);
    lse_merge(m[t], z[t], mo, zo);
  }
  __syncthreads();  // the query tiles are no longer read
  float2* red = (float2*)qs;  // [NW][NQ*32]
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) red[wave * NQ * 32 + t * 32 + lane] = make_float2(m[t], z[t]);
  }
  __syncthreads();
  for (int r = tid; r < nrows; r += NT) {
    float mm = -INFINITY, zz = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float2 pz = red[w * NQ * 32 + r];
      lse_merge(mm, zz, pz.x, pz.y);
    }
    a.part[((size_t)head * a.GWr + row0 + r) * a.nchunk + chunk] = make_float2(mm, zz);
  }
}

template <int D, int NQ, int NW>
__global__ void __launch_bounds__(NW * 64) score_pass2_32(ScoreArgs a) {
  constexpr int NV = D / 16;
  constexpr int NT = NW * 64;
  __shared__ u32x4_t qs[NQ * NV * 64];
  __shared__ float ls[NQ * 32];
  __shared__ int lims[NQ * 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, head = blockIdx.y, grp = blockIdx.z;
  const int b = head / a.Hkv, hk = head - b * a.Hkv;
  const int row0 = grp * a.qcap;
  const int nrows = min(a.qcap, a.GW - row0);
  const int S = a.S;
  const float c = a.c;
  const char* kh = (const char*)((const uint16_t*)a.k + (size_t)head * a.kstride * D);
  const int k0 = chunk * a.chunk;
  const int kend = min(S, k0 + a.chunk);
  const int mask_from = a.causal ? (S - a.W + 1) : S;

  int kb = k0 + wave * 64;
  Frag<NV> kf[2];
  if (kb < kend) load_key_block32<D>(kf, kh, kb, S, lane);
  // No combine launch: this workgroup merges its rows' chunk statistics,
  // their loads in flight with the keys and queries.
  const bool fold = a.fold_tl >= 0;
  FoldRows<NT, NQ * 32> fr;
  if (fold) fr.load(a.part + ((size_t)head * a.GWr + row0) * a.nchunk, a.nchunk, a.fold_tl, nrows);
  const uint16_t* qg = (const uint16_t*)a.q + ((size_t)(b * a.Hq + hk * a.G) * a.W + row0) * D;
  stage_queries32<D, NT>(qs, qg, nrows, NQ);
  for (int r = tid; r < NQ * 32; r += NT) {
    // rows past the group's end get an infinite normaliser (weight 0)
    ls[r] = (r < nrows && !fold) ? a.lse[(size_t)head * a.GWr + row0 + r] : INFINITY;
    lims[r] = key_limit(a, row0 + r);
  }
  if (fold) {
    __syncthreads();
    fr.merge(a.nchunk, a.fold_tl, nrows, ls);
  }
  __shared__ int prog[NW];
  if (tid < NW) prog[tid] = 0;
  int nblk = 0;
  __syncthreads();

  float* out = a.s_out + ((size_t)grp * gridDim.y + head) * S;
  for (; kb < kend; kb += NW * 64) {
    int lds_off = 0;
    asm volatile("" : "+v"(lds_off));
    const u32x4_t* qsv = qs + lds_off;
    const float* lsv = ls + lds_off;
    float as[2] = {0.f, 0.f};
    if (kb + 64 > mask_from)
      pass2_block32<NV, NQ, true>(lims, kf, qsv, lsv, as, kb, lane, c);
    else
      pass2_block32<NV, NQ, false>(lims, kf, qsv, lsv, as, kb, lane, c);
    as[0] += __shfl_xor(as[0], 32);
    as[1] += __shfl_xor(as[1], 32);
    // lane l writes key kb + l: key tile l / 32, column l % 32.  The store
    // goes out before the next block's key loads, so waiting for those keys
    // (the vector-memory counter counts stores too) never waits for it.
    const float mine = (lane >> 5) ? as[1] : as[0];
    if (kb + lane < kend) out[kb + lane] = mine;
    if (kb + NW * 64 < kend) load_key_block32<D>(kf, kh, kb + NW * 64, S, lane);
    pace_partner<NW>(prog, wave, lane, nblk);
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// Keys in LDS, query rows streamed: for scoring without a causal mask over a
// few keys by many query rows (Kara's decode window: G*|W| = 2048 rows per
// KV head against its 448 compressible keys).  One workgroup per KV head
// holds the head's S keys (a multiple of 32, at most 512) in LDS in fragment
// order.  Each wave takes 32-row query tiles straight from memory into
// registers and, with the same fragments, first finds each row's max and
// log2-sum-exp over all keys (keys on the matrix rows: one row per lane),
// then adds the row's normalised weights into per-key column sums kept in
// registers (rows on the matrix rows: one key per lane).  The waves' column
// sums are added in wave order at the end.  Every key row and every query row is read once; there
// are no per-chunk statistics and no combine launch.
constexpr int kKsMaxKeyTiles = 16;   // up to 512 keys
constexpr int kKsWaves = 8;

template <int D, int NKT>
__global__ void __launch_bounds__(kKsWaves * 64) score_keys_lds32(ScoreArgs a) {
  constexpr int NV = D / 16, NW = kKsWaves, NT = NW * 64;
  static_assert(NKT >= 1 && NKT <= kKsMaxKeyTiles, "key tiles");
  __shared__ u32x4_t kl[NKT * NV * 64];   // key tile kt, fragment v, lane
  __shared__ float csum[NW][NKT * 32];    // each wave's column sums
  __shared__ __attribute__((aligned(16))) float lsw[NW][32];   // a tile's row normalisers
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int head = blockIdx.x, b = head / a.Hkv, hk = head - b * a.Hkv;
  const int S = a.S, GW = a.GW;   // S == 32 * NKT: no key is masked
  const float c = a.c;
  if (a.zero) {
    // the select that follows finds its histograms cleared
    for (long i = (long)head * NT + tid; i < a.zero_words; i += (long)gridDim.x * NT)
      a.zero[i] = 0u;
  }
  const char* kh = (const char*)((const uint16_t*)a.k + (size_t)head * a.kstride * D);
  for (int tv = wave; tv < NKT * NV; tv += NW) {
    const int kt = tv / NV, v = tv - kt * NV;
    const int row = kt * 32 + r;
    const char* src = kh + (size_t)row * (D * 2) + h * D + 16 * v;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)(kl + tv * 64),
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const uint16_t* qg = (const uint16_t*)a.q + (size_t)(b * a.Hq + hk * a.G) * a.W * D;
  // Key fragments are read from LDS at every use: each pass reads them
  // through its own opaque copy of the base, or the compiler would keep the
  // first pass's fragments of every tile in registers for the second.
  auto kfrag = [&](const u32x4_t* base, int kt) {
    Frag<NV> f;
#pragma unroll
    for (int i = 0; i < NV; ++i) f.v[i] = base[(kt * NV + i) * 64 + lane];
    return f;
  };
  float cs[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) cs[kt] = 0.f;
  const int ntq = (GW + 31) / 32;
  for (int t = wave; t < ntq; t += NW) {
    Frag<NV> qf;
    {
      const int row = min(t * 32 + r, GW - 1);
      const char* src = (const char*)(qg + (size_t)row * D) + h * D;
#pragma unroll
      for (int i = 0; i < NV; ++i) qf.v[i] = *(const u32x4_t*)(src + 16 * i);
    }
    // First pass: cur[i] is key kt*32 + 8*(i/4) + 4h + i%4 of query row r.
    float m = -INFINITY, z = 0.f;
    {
      int off = 0;
      asm volatile("" : "+v"(off));
      const u32x4_t* k1 = kl + off;
      f32x16_t acc[2];
      acc[0] = mma32<NV>(kfrag(k1, 0), qf, zero16());
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        f32x16_t& cur = acc[kt & 1];
        if (kt + 1 < NKT) acc[(kt + 1) & 1] = mma32<NV>(kfrag(k1, kt + 1), qf, zero16());
        const float mnew = fmaxf(m, max16(cur) * c);
        const float mu = (mnew == -INFINITY) ? 0.f : mnew;
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(cur[i], c, -mu));
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
          for (int i = 0; i < w; ++i) e[i] += e[i + w];
        z = fmaf(z, __builtin_amdgcn_exp2f(m - mu), e[0]);
        m = mnew;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Lanes r and r + 32 hold the two key halves of row r.
    lse_merge(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
    // rows past the group's end get an infinite normaliser (weight 0)
    if (h == 0) lsw[wave][r] = (t * 32 + r < GW) ? m + log2f(z) : INFINITY;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t lq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lq[j] = *(const f32x4_t*)&lsw[wave][8 * j + 4 * h];
    // Second pass: cur[i] is query row 8*(i/4) + 4h + i%4 of key kt*32 + r.
    {
      int off = 0;
      asm volatile("" : "+v"(off));
      const u32x4_t* k2 = kl + off;
      f32x16_t acc[2];
      acc[0] = mma32<NV>(qf, kfrag(k2, 0), zero16());
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        f32x16_t& cur = acc[kt & 1];
        if (kt + 1 < NKT) acc[(kt + 1) & 1] = mma32<NV>(qf, kfrag(k2, kt + 1), zero16());
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          e[i] = __builtin_amdgcn_exp2f(fmaf(cur[i], c, -lq[i >> 2][i & 3]));
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
          for (int i = 0; i < w; ++i) e[i] += e[i + w];
        cs[kt] += e[0];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lsw is rewritten by the next tile only after every lane read it
    __builtin_amdgcn_wave_barrier();
  }
  // Lanes r and r + 32 hold the two row halves of key kt*32 + r.
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const float v = cs[kt] + __shfl_xor(cs[kt], 32);
    if (h == 0) csum[wave][kt * 32 + r] = v;
  }
  __syncthreads();
  float* out = a.s_out + (size_t)head * S;
  for (int j = tid; j < S; j += NT) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += csum[w][j];
    out[j] = v;
  }
}

// ---------------------------------------------------------------------------
// Pass 2 with the streaming top-k of TideKV Algorithm 2 (the heap of pass 2):
// no per-key score vector leaves the workgroup.  A workgroup computes the
// raw scores of its key chunk plus one 64-key block on either side (the
// halo the max filter needs) into LDS, pools them there, and keeps the
// top-`budget` pooled candidates of the chunk (all of them when the chunk
// has fewer), which it writes in ascending position order to its slot of a
// per-row candidate list.  The global top-budget is a subset of the union of
// the chunk lists, so a selection over the lists (ties to the lower list
// index, which is the lower position) finishes the job.  Scratch is
// O(chunks x budget) per row, independent of S while the chunk count is
// fixed by the machine.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxChunk = 16384;

// Candidates of chunk c: [max(lo, c*chunk), min(hi, (c+1)*chunk)).
__device__ __forceinline__ int chunk_candidates(int c, int chunk, int lo, int hi) {
  return max(0, min(hi, (c + 1) * chunk) - max(lo, c * chunk));
}

template <int D, int NQ, int NW>
__global__ void __launch_bounds__(NW * 64) score_pass2_stream(ScoreArgs a, StreamArgs sa) {
  constexpr int NV = D / 16;
  constexpr int NT = NW * 64;
  constexpr int PER = kStreamMaxChunk / NT;
  __shared__ u32x4_t qs[NQ * NV * 64];
  __shared__ float ls[NQ * 32];
  __shared__ int lims[NQ * 32];
  extern __shared__ float sc[];   // a.chunk + 128 scores (dynamic)
  __shared__ __attribute__((aligned(16))) uint32_t hist[2048];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t pick[3];
  __shared__ int off_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, head = blockIdx.y;
  const int b = head / a.Hkv, hk = head - b * a.Hkv;
  const int nrows = min(a.qcap, a.GW);
  const int S = a.S;
  const float c = a.c;
  const char* kh = (const char*)((const uint16_t*)a.k + (size_t)head * a.kstride * D);
  const int k0 = chunk * a.chunk;
  const int kend = min(S, k0 + a.chunk);
  const int x0 = k0 >= 64 ? k0 - 64 : 0;        // chunk with a one-block halo
  const int x1 = min(S, kend + 64);
  const int mask_from = a.causal ? (S - a.W + 1) : S;

  int kb = x0 + wave * 64;
  Frag<NV> kf[2];
  if (kb < x1) load_key_block32<D>(kf, kh, kb, S, lane);
  const uint16_t* qg = (const uint16_t*)a.q + ((size_t)(b * a.Hq + hk * a.G) * a.W) * D;
  stage_queries32<D, NT>(qs, qg, nrows, NQ);
  for (int r = tid; r < NQ * 32; r += NT) {
    ls[r] = (r < nrows) ? a.lse[(size_t)head * a.GWr + r] : INFINITY;
    lims[r] = key_limit(a, r);
  }
  if (tid == 0) {
    int off = 0;
    for (int cc = 0; cc < chunk; ++cc) off += min(sa.budget, chunk_candidates(cc, a.chunk, sa.lo, sa.hi));
    off_s = off;
  }
  __syncthreads();
  for (; kb < x1; kb += NT) {
    float as[2] = {0.f, 0.f};
    if (kb + 64 > mask_from) pass2_block32<NV, NQ, true>(lims, kf, qs, ls, as, kb, lane, c);
    else pass2_block32<NV, NQ, false>(lims, kf, qs, ls, as, kb, lane, c);
    if (kb + NT < x1) load_key_block32<D>(kf, kh, kb + NT, S, lane);
    as[0] += __shfl_xor(as[0], 32);
    as[1] += __shfl_xor(as[1], 32);
    const float mine = (lane >> 5) ? as[1] : as[0];
    if (kb + lane < x1) sc[kb - x0 + lane] = mine;
  }
  __syncthreads();
  // Max filter over the candidate range, into registers, then in place.
  const int c0 = max(sa.lo, k0), c1 = min(sa.hi, kend);
  const int nc = max(0, c1 - c0);
  float pv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = c0 + j * NT + tid;
    float m = 0.f;
    if (i < c1) {
      const int j0 = max(sa.lo, i - sa.ph), j1 = min(sa.hi - 1, i + sa.ph);
      m = sc[j0 - x0];
      for (int t = j0 + 1; t <= j1; ++t) m = fmaxf(m, sc[t - x0]);
    }
    pv[j] = m;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (j * NT + tid < nc) sc[j * NT + tid] = pv[j];
  __syncthreads();
  const int keep = min(sa.budget, nc);
  if (keep == 0) return;
  float* dv = sa.cval + (size_t)head * sa.M + off_s;
  int32_t* dp = sa.cpos + (size_t)head * sa.M + off_s;
  if (nc <= sa.budget) {
    for (int i = tid; i < nc; i += NT) {
      dv[i] = sc[i];
      dp[i] = c0 + i;
    }
    return;
  }
  // Exact top-keep of the chunk: radix select on the bit patterns (scores
  // are >= 0, so bit order is value order), ties to the lower position.
  const uint32_t* sb = (const uint32_t*)sc;
  uint32_t prefix = 0u, pmask = 0u, rem = (uint32_t)keep;
  for (int r = 0; r < 3; ++r) {
    const int shift = r == 0 ? 20 : (r == 1 ? 10 : 0);
    const int nb = r == 0 ? 2048 : 1024;
    for (int i = tid; i < nb; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nc; i += NT) {
      const uint32_t x = sb[i];
      hist_add(hist, (x >> shift) & (uint32_t)(nb - 1), (x & pmask) == prefix);
    }
    __syncthreads();
    if (r == 0) block_find_digit<2048>(hist, rem, pick);
    else block_find_digit<1024>(hist, rem, pick);
    rem -= pick[1];
    prefix |= pick[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    const bool whole = rem == pick[2];
    __syncthreads();
    if (whole) break;
  }
  // Ordered write: kept = above the prefix, or equal to it among the first
  // `rem` equal ones in position order.
  uint32_t out_base = 0u, eq_base = 0u;
  for (int i0 = 0; i0 < nc; i0 += NT) {
    const int i = i0 + tid;
    const uint32_t x = i < nc ? sb[i] : 0u;
    const uint32_t km = x & pmask;
    const bool gt = i < nc && km > prefix;
    const bool eq = i < nc && km == prefix;
    uint32_t eq_tot;
    const uint32_t eq_before = eq_base + block_exclusive_scan<NT>(eq ? 1u : 0u, &eq_tot, wsum);
    const bool kp = gt || (eq && eq_before < rem);
    uint32_t kp_tot;
    const uint32_t slot = out_base + block_exclusive_scan<NT>(kp ? 1u : 0u, &kp_tot, wsum);
    if (kp && slot < (uint32_t)keep) {
      dv[slot] = __uint_as_float(x);
      dp[slot] = c0 + i;
    }
    out_base += kp_tot;
    eq_base += eq_tot;
  }
}

// ---------------------------------------------------------------------------
// Combine the per-chunk partials of each query row: lse = max + log2(sum).
// 2^tpr_log2 consecutive lanes share a row (just enough for about four
// partials each, so short chunk lists do not leave a wave per row mostly
// idle); each lane merges its strided partials in order, then a fixed
// butterfly merges the lanes.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) score_combine(const float2* __restrict__ part,
                                                     float* __restrict__ lse, int nheads,
                                                     int nchunk, int GW, int GWr, int tpr_log2,
                                                     uint32_t* __restrict__ zero,
                                                     long zero_words) {
  const int tpr = 1 << tpr_log2;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  for (long i = gid; i < zero_words; i += (long)gridDim.x * 256) zero[i] = 0u;
  const long row_id = gid >> tpr_log2;
  const int sub = (int)(gid & (tpr - 1));
  const bool valid = row_id < (long)nheads * GW;
  const int head = valid ? (int)(row_id / GW) : 0;
  const int r = valid ? (int)(row_id - (long)head * GW) : 0;
  float m = -INFINITY, z = 0.f;
  if (valid) {
    // A lane's partials, in chunk order, read CB at a time with all CB loads
    // in flight before the first merge.
    constexpr int CB = 4;
    const float2* p = part + ((size_t)head * GWr + r) * nchunk;
    for (int ch0 = sub; ch0 < nchunk; ch0 += CB * tpr) {
      float2 pz[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) pz[j] = p[min(ch0 + j * tpr, nchunk - 1)];
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (ch0 + j * tpr < nchunk) lse_merge(m, z, pz[j].x, pz[j].y);
    }
  }
  for (int off = tpr >> 1; off >= 1; off >>= 1) {
    const float mo = __shfl_xor(m, off);
    const float zo = __shfl_xor(z, off);
    lse_merge(m, z, mo, zo);
  }
  if (valid && sub == 0) lse[(size_t)head * GWr + r] = m + log2f(z);
}

// ---------------------------------------------------------------------------
// Pass 2: s[key] = sum over the group's query rows of exp2(l*c - lse[row]).
// ---------------------------------------------------------------------------
template <typename T, int D, int NQT, int NW>
__global__ void __launch_bounds__(NW * 64) score_pass2(ScoreArgs a) {
  constexpr int NV = nvec<T, D>();
  constexpr int NT = NW * 64;
  constexpr int RB = D * (int)sizeof(T);
  __shared__ u32x4_t qs[NQT * NV * 64];
  __shared__ float ls[NQT * 16];
  __shared__ int lims[NQT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int chunk = blockIdx.x, head = blockIdx.y, grp = blockIdx.z;
  const int b = head / a.Hkv, hk = head - b * a.Hkv;
  const int row0 = grp * a.qcap;
  const int nrows = min(a.qcap, a.GW - row0);
  const int S = a.S;
  const float c = a.c;
  const char* kh = (const char*)((const T*)a.k + (size_t)head * a.kstride * D);
  const int k0 = chunk * a.chunk;
  const int kend = min(S, k0 + a.chunk);
  const int mask_from = a.causal ? (S - a.W + 1) : S;

  int kb = k0 + wave * 64;
  Frag<NV> kf[4];
  if (kb < kend) load_key_block<NV>(kf, kh, kb, S, RB, l16, g);
  const T* qg = (const T*)a.q + ((size_t)(b * a.Hq + hk * a.G) * a.W + row0) * D;
  stage_queries<T, D, NT>(qs, qg, nrows, NQT);
  for (int r = tid; r < NQT * 16; r += NT) {
    ls[r] = (r < nrows) ? a.lse[(size_t)head * a.GWr + row0 + r] : INFINITY;
    lims[r] = key_limit(a, row0 + r);
  }
  __syncthreads();

  float* out = a.s_out + ((size_t)grp * gridDim.y + head) * S;
  for (; kb < kend; kb += NW * 64) {
    Frag<NV> kn[4];
    const bool has_next = kb + NW * 64 < kend;
    if (has_next) load_key_block<NV>(kn, kh, kb + NW * 64, S, RB, l16, g);
    int lds_off = 0;
    asm volatile("" : "+v"(lds_off));
    const u32x4_t* qsv = qs + lds_off;
    const float* lsv = ls + lds_off;
    float as[4] = {0.f, 0.f, 0.f, 0.f};
    if (kb + 64 > mask_from)
      pass2_block<T, NV, NQT, true>(lims, kf, qsv, lsv, as, kb, row0, lane, g, l16, c);
    else
      pass2_block<T, NV, NQT, false>(lims, kf, qsv, lsv, as, kb, row0, lane, g, l16, c);
    if (has_next) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = kn[kt];
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      as[kt] += __shfl_xor(as[kt], 16);
      as[kt] += __shfl_xor(as[kt], 32);
    }
    const float mine = g == 0 ? as[0] : (g == 1 ? as[1] : (g == 2 ? as[2] : as[3]));
    const int key = kb + g * 16 + l16;
    if (key < kend) out[key] = mine;
  }
}

// Sum the per-group partial scores in group order (only when ngroups > 1).
__global__ void __launch_bounds__(256) score_group_sum(const float* __restrict__ sg,
                                                       float* __restrict__ s, size_t n,
                                                       int ngroups) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = sg[i];
  for (int gi = 1; gi < ngroups; ++gi) v += sg[(size_t)gi * n + i];
  s[i] = v;
}

// p[i] = max of s[j], j in [i-h, i+h] within the candidates [lo, hi); 0 outside.
__global__ void __launch_bounds__(256) maxpool_kernel(const float* __restrict__ s,
                                                   float* __restrict__ p, int S, int lo, int hi,
                                                   int h) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= S) return;
  const size_t base = (size_t)blockIdx.y * S;
  float v = 0.f;
  if (i >= lo && i < hi) {
    const int j0 = max(lo, i - h), j1 = min(hi - 1, i + h);
    v = s[base + j0];
    for (int j = j0 + 1; j <= j1; ++j) v = fmaxf(v, s[base + j]);
  }
  p[base + i] = v;
}

template <typename T, int D, int NQT, int NW>
void launch_passes(const ScoreArgs& args, dim3 grid, hipStream_t stream, const ScorePlan& p) {
  KVSEL_LAUNCH("score_pass1", (score_pass1<T, D, NQT, NW>), grid, dim3(NW * 64), 0, stream, args);
  int tl = 0;
  while ((4 << tl) < p.nchunk && tl < 6) ++tl;
  const long lanes = ((long)p.nheads * p.GW) << tl;
  KVSEL_LAUNCH("score_combine", score_combine, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream,
                     args.part, args.lse, p.nheads, p.nchunk, p.GW, p.GWr, tl, args.zero,
               args.zero_words);
  KVSEL_LAUNCH("score_pass2", (score_pass2<T, D, NQT, NW>), grid, dim3(NW * 64), 0, stream, args);
}

template <int D, int NQ, int NW>
void launch_passes32(const ScoreArgs& args, dim3 grid, hipStream_t stream, const ScorePlan& p) {
  KVSEL_LAUNCH("score_pass1_32", (score_pass1_32<D, NQ, NW>), grid, dim3(NW * 64), 0, stream, args);
  if (args.fold_tl >= 0) {
    KVSEL_LAUNCH("score_pass2_32", (score_pass2_32<D, NQ, NW>), grid, dim3(NW * 64), 0, stream,
                 args);
    return;
  }
  int tl = 0;
  while ((4 << tl) < p.nchunk && tl < 6) ++tl;
  const long lanes = ((long)p.nheads * p.GW) << tl;
  KVSEL_LAUNCH("score_combine", score_combine, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream,
                     args.part, args.lse, p.nheads, p.nchunk, p.GW, p.GWr, tl, args.zero,
               args.zero_words);
  KVSEL_LAUNCH("score_pass2_32", (score_pass2_32<D, NQ, NW>), grid, dim3(NW * 64), 0, stream, args);
}

template <int D>
bool dispatch_qt32(int nq, const ScoreArgs& args, dim3 grid, hipStream_t stream,
                   const ScorePlan& p) {
  switch (nq) {
    case 1: launch_passes32<D, 1, 4>(args, grid, stream, p); return true;
    case 2: launch_passes32<D, 2, 4>(args, grid, stream, p); return true;
    case 4: launch_passes32<D, 4, 4>(args, grid, stream, p); return true;
    case 8: launch_passes32<D, 8, 4>(args, grid, stream, p); return true;
    case 10: launch_passes32<D, 10, 8>(args, grid, stream, p); return true;
    case 16: launch_passes32<D, 16, 8>(args, grid, stream, p); return true;
    default: return false;
  }
}

template <typename T, int D>
bool dispatch_qt(int nqt, const ScoreArgs& args, dim3 grid, hipStream_t stream,
                 const ScorePlan& p) {
  switch (nqt) {
    case 1: launch_passes<T, D, 1, 4>(args, grid, stream, p); return true;
    case 2: launch_passes<T, D, 2, 4>(args, grid, stream, p); return true;
    case 4: launch_passes<T, D, 4, 4>(args, grid, stream, p); return true;
    case 8: launch_passes<T, D, 8, 4>(args, grid, stream, p); return true;
    case 16: launch_passes<T, D, 16, 4>(args, grid, stream, p); return true;
    case 20:
      if constexpr (nvec<T, D>() <= 4) {
        launch_passes<T, D, 20, 8>(args, grid, stream, p);
        return true;
      }
      return false;
    default: return false;
  }
}

}  // namespace

static bool plan_chunks(const kvsel_desc& d, ScorePlan* p, int lds_bytes);

bool plan_score(const kvsel_desc& d, ScorePlan* p) {
  const int e = d.dtype == KVSEL_F32 ? 4 : 2;
  const int tile_bytes = 16 * d.head_dim * e;
  p->nheads = d.batch * d.n_kv_heads;
  p->G = d.n_q_heads / d.n_kv_heads;
  p->GW = p->G * d.obs_window;
  p->GWr = (p->GW + 15) / 16 * 16;
  const int nqt = p->GWr / 16;
  // Query tiles per workgroup: the whole group, rounded up to a built tile
  // count, when it fits in about 80 KiB of LDS (20 tiles of 4 KiB run 8 waves
  // per workgroup, one workgroup per CU); otherwise groups of 16 tiles, each
  // re-reading its key chunk.
  // 32x32 tiles for bf16 prompts of 4096 keys or more; the 16x16 form is
  // faster on short key ranges (the 448-key decode window: 304 vs 353 us).
  // No causal mask, few keys, many query rows (a decode window scoring its
  // own keys): one workgroup per KV head with the keys in LDS.
  p->keys_lds = d.dtype == KVSEL_BF16 && !d.causal && d.seq_len <= kKsMaxKeyTiles * 32 &&
                d.seq_len % 32 == 0 && p->GW >= 256 && (d.head_dim == 64 || d.head_dim == 128);
  p->mfma32 = d.dtype == KVSEL_BF16 && d.seq_len >= 4096;
  if (p->mfma32) {
    // 32-row tiles: the whole group when it fits 10 tiles (8 waves), else
    // groups of 16 tiles (8 waves, 128 KiB of LDS at D = 128: fewer groups
    // re-reading each key chunk); 32*D*2 bytes of LDS per tile.
    const int nq = (p->GW + 31) / 32;
    const int maxq = nq <= 1 ? 1 : nq <= 2 ? 2 : nq <= 4 ? 4 : nq <= 8 ? 8 : nq <= 10 ? 10 : 16;
    p->maxqt = maxq;
    p->nwaves = maxq >= 10 ? 8 : 4;
    p->qcap = 32 * maxq;
    p->ngroups = (p->GW + p->qcap - 1) / p->qcap;
    return plan_chunks(d, p, maxq * 32 * d.head_dim * 2 + maxq * 32 * 8);
  }
  int maxqt;
  if (nqt <= 1) maxqt = 1;
  else if (nqt <= 2) maxqt = 2;
  else if (nqt <= 4) maxqt = 4;
  else if (nqt <= 8) maxqt = 8;
  else if (nqt <= 16) maxqt = 16;
  else if (nqt <= 20 && tile_bytes <= 4096) maxqt = 20;
  else maxqt = 16;
  if (tile_bytes > 4096 && maxqt > 8) maxqt = 8;
  p->maxqt = maxqt;
  p->nwaves = (maxqt == 20) ? 8 : 4;
  p->qcap = 16 * maxqt;
  p->ngroups = (p->GW + p->qcap - 1) / p->qcap;
  return plan_chunks(d, p, maxqt * tile_bytes + maxqt * 16 * 8);
}

// Chunk statistics (rows x chunks) up to which pass 2 merges them itself:
// the 8K layer's 128 rows x 32 chunks, 32 KiB of L2 reads per workgroup.
constexpr long kFoldMaxPartials = 4096;

// Key chunks and the workspace layout for a plan whose tiles are chosen.
static bool plan_chunks(const kvsel_desc& d, ScorePlan* p, int lds_bytes) {
  // Key chunk: a multiple of one workgroup step, sized so the grid is about
  // one full wave of resident workgroups (fewer, longer workgroups amortise
  // the query staging and keep the key prefetch busy).
  const int step = p->nwaves * 64;
  int wg_per_cu = (160 * 1024) / lds_bytes;
  const int wave_cap = 8 / p->nwaves;     // about two waves per SIMD
  if (wg_per_cu > wave_cap) wg_per_cu = wave_cap;
  if (wg_per_cu < 1) wg_per_cu = 1;
  const long target_wg = 256L * wg_per_cu;
  const long wg_per_chunk = (long)p->nheads * p->ngroups;
  long want_chunks = (target_wg + wg_per_chunk - 1) / wg_per_chunk;
  if (want_chunks < 1) want_chunks = 1;
  long steps = ((long)d.seq_len + (long)step * want_chunks - 1) / ((long)step * want_chunks);
  if (steps < 1) steps = 1;
  p->chunk = (int)(steps * step);
  p->nchunk = (d.seq_len + p->chunk - 1) / p->chunk;
  // Few rows and chunks: every pass-2 workgroup merges its rows' chunk
  // statistics (at most kFoldMaxPartials reads from the L2) rather than
  // waiting for a combine launch.
  p->fold_tl = -1;
  if (p->mfma32 && p->ngroups == 1 && (long)p->GW * p->nchunk <= kFoldMaxPartials) {
    // the combine's lanes per row: the fewest with 4 << tl >= nchunk
    int tl = 0;
    while ((4 << tl) < p->nchunk && tl < 6) ++tl;
    if (tl <= 3) p->fold_tl = tl;
  }
  size_t off = 0;
  p->off_part = off;
  off = align256(off + (size_t)p->nheads * p->nchunk * p->GWr * sizeof(float2));
  p->off_lse = off;
  off = align256(off + (size_t)p->nheads * p->GWr * sizeof(float));
  p->off_raw = off;
  off = align256(off + (size_t)p->nheads * d.seq_len * sizeof(float));
  p->off_grp = off;
  if (p->ngroups > 1) off = align256(off + (size_t)p->ngroups * p->nheads * d.seq_len * sizeof(float));
  p->total = off;
  if (p->keys_lds) {
    // one launch with no per-chunk statistics: only the raw score vector
    p->off_part = p->off_lse = p->off_grp = p->off_raw = 0;
    p->total = align256((size_t)p->nheads * d.seq_len * sizeof(float));
  }
  return true;
}

template <int D, int NKT>
static void launch_keys_lds(const ScoreArgs& a, int nheads, hipStream_t stream) {
  KVSEL_LAUNCH("score_keys_lds32", (score_keys_lds32<D, NKT>), dim3(nheads), dim3(kKsWaves * 64),
               0, stream, a);
}

// The keys-in-LDS scoring for S keys (a multiple of 32): the kernel built for
// S / 32 tiles.
template <int D>
static bool dispatch_keys_lds(int S, const ScoreArgs& a, int nheads, hipStream_t stream) {
  if (S % 32 != 0) return false;
  switch (S / 32) {
    case 1: launch_keys_lds<D, 1>(a, nheads, stream); return true;
    case 2: launch_keys_lds<D, 2>(a, nheads, stream); return true;
    case 3: launch_keys_lds<D, 3>(a, nheads, stream); return true;
    case 4: launch_keys_lds<D, 4>(a, nheads, stream); return true;
    case 5: launch_keys_lds<D, 5>(a, nheads, stream); return true;
    case 6: launch_keys_lds<D, 6>(a, nheads, stream); return true;
    case 7: launch_keys_lds<D, 7>(a, nheads, stream); return true;
    case 8: launch_keys_lds<D, 8>(a, nheads, stream); return true;
    case 9: launch_keys_lds<D, 9>(a, nheads, stream); return true;
    case 10: launch_keys_lds<D, 10>(a, nheads, stream); return true;
    case 11: launch_keys_lds<D, 11>(a, nheads, stream); return true;
    case 12: launch_keys_lds<D, 12>(a, nheads, stream); return true;
    case 13: launch_keys_lds<D, 13>(a, nheads, stream); return true;
    case 14: launch_keys_lds<D, 14>(a, nheads, stream); return true;
    case 15: launch_keys_lds<D, 15>(a, nheads, stream); return true;
    case 16: launch_keys_lds<D, 16>(a, nheads, stream); return true;
    default: return false;
  }
}

kvsel_status launch_score(const kvsel_desc& d, const ScorePlan& p, const void* q, const void* k,
                          float* raw, float* pooled, int pool_kernel, char* ws,
                          hipStream_t stream, int kstride, uint32_t* zero, size_t zero_words) {
  ScoreArgs a;
  a.zero = zero;
  a.zero_words = (long)zero_words;
  a.q = q;
  a.k = k;
  a.part = (float2*)(ws + p.off_part);
  a.lse = (float*)(ws + p.off_lse);
  float* s = raw ? raw : (float*)(ws + p.off_raw);
  a.s_out = p.ngroups > 1 ? (float*)(ws + p.off_grp) : s;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.G = p.G;
  a.W = d.obs_window;
  a.S = d.seq_len;
  a.kstride = kstride;
  a.GW = p.GW;
  a.GWr = p.GWr;
  a.qcap = p.qcap;
  a.chunk = p.chunk;
  a.nchunk = p.nchunk;
  a.causal = d.causal;
  // KVSEL_SCORE_COMBINE=1 (debugging): the combine launch for every plan
  const char* force = getenv("KVSEL_SCORE_COMBINE");
  const bool combine = force && force[0] && strcmp(force, "0") != 0;
  a.fold_tl = (p.mfma32 && !combine) ? p.fold_tl : -1;
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.head_dim);
  a.c = scale * kLog2e;
  const dim3 grid(p.nchunk, p.nheads, p.ngroups);
  bool ok = false;
  if (p.keys_lds) {
    a.s_out = s;
    ok = d.head_dim == 128 ? dispatch_keys_lds<128>(d.seq_len, a, p.nheads, stream)
                           : dispatch_keys_lds<64>(d.seq_len, a, p.nheads, stream);
  } else if (p.mfma32) {
    ok = d.head_dim == 128 ? dispatch_qt32<128>(p.maxqt, a, grid, stream, p)
                           : dispatch_qt32<64>(p.maxqt, a, grid, stream, p);
  } else if (d.dtype == KVSEL_BF16) {
    ok = d.head_dim == 128 ? dispatch_qt<uint16_t, 128>(p.maxqt, a, grid, stream, p)
                           : dispatch_qt<uint16_t, 64>(p.maxqt, a, grid, stream, p);
  } else {
    ok = d.head_dim == 128 ? dispatch_qt<float, 128>(p.maxqt, a, grid, stream, p)
                           : dispatch_qt<float, 64>(p.maxqt, a, grid, stream, p);
  }
  if (!ok) return KVSEL_ERR_UNSUPPORTED;
  if (p.ngroups > 1 && !p.keys_lds) {
    const size_t n = (size_t)p.nheads * d.seq_len;
    KVSEL_LAUNCH("score_group_sum", score_group_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a.s_out, s, n, p.ngroups);
  }
  if (!pooled) return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
  const int lo = d.n_sink, hi = d.seq_len - d.obs_window;
  KVSEL_LAUNCH("maxpool_kernel", maxpool_kernel, dim3((d.seq_len + 255) / 256, p.nheads), dim3(256), 0, stream,
                     s, pooled, d.seq_len, lo, hi, (pool_kernel - 1) / 2);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

bool plan_score_stream(const kvsel_desc& d, ScorePlan* p) {
  if (!plan_score(d, p) || !p->mfma32 || p->ngroups != 1 || p->maxqt > 10) return false;
  // A chunk is held in LDS next to the query tiles.
  return p->chunk <= kStreamMaxChunk;
}

int stream_list_len(const ScorePlan& p, int lo, int hi, int budget) {
  int m = 0;
  for (int c = 0; c < p.nchunk; ++c) {
    const int n = std::max(0, std::min(hi, (c + 1) * p.chunk) - std::max(lo, c * p.chunk));
    m += std::min(budget, n);
  }
  return m;
}

template <int D, int NQ, int NW>
static void launch_stream_passes(const ScoreArgs& args, const StreamArgs& sa, dim3 grid,
                                 hipStream_t stream, const ScorePlan& p) {
  KVSEL_LAUNCH("score_pass1_32", (score_pass1_32<D, NQ, NW>), grid, dim3(NW * 64), 0, stream,
               args);
  int tl = 0;
  while ((4 << tl) < p.nchunk && tl < 6) ++tl;
  const long lanes = ((long)p.nheads * p.GW) << tl;
  KVSEL_LAUNCH("score_combine", score_combine, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0,
               stream, args.part, args.lse, p.nheads, p.nchunk, p.GW, p.GWr, tl, args.zero,
               args.zero_words);
  const size_t lds = (size_t)(p.chunk + 128) * sizeof(float);
  KVSEL_LAUNCH("score_pass2_stream", (score_pass2_stream<D, NQ, NW>), grid, dim3(NW * 64), lds,
               stream, args, sa);
}

kvsel_status launch_score_stream(const kvsel_desc& d, const ScorePlan& p, const void* q,
                                 const void* k, const StreamArgs& sa, char* ws,
                                 hipStream_t stream) {
  ScoreArgs a;
  a.q = q;
  a.k = k;
  a.part = (float2*)(ws + p.off_part);
  a.lse = (float*)(ws + p.off_lse);
  a.s_out = nullptr;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.G = p.G;
  a.W = d.obs_window;
  a.S = d.seq_len;
  a.kstride = d.seq_len;
  a.GW = p.GW;
  a.GWr = p.GWr;
  a.qcap = p.qcap;
  a.chunk = p.chunk;
  a.nchunk = p.nchunk;
  a.causal = d.causal;
  a.zero = nullptr;
  a.zero_words = 0;
  a.fold_tl = -1;   // the streaming pass 2 reads lse from the combine
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.head_dim);
  a.c = scale * kLog2e;
  const dim3 grid(p.nchunk, p.nheads, 1);
  const int nq = p.maxqt;
#define KVSEL_STREAM(DD, NQQ, NWW) launch_stream_passes<DD, NQQ, NWW>(a, sa, grid, stream, p)
  if (d.head_dim == 128) {
    switch (nq) {
      case 1: KVSEL_STREAM(128, 1, 4); break;
      case 2: KVSEL_STREAM(128, 2, 4); break;
      case 4: KVSEL_STREAM(128, 4, 4); break;
      case 8: KVSEL_STREAM(128, 8, 4); break;
      case 10: KVSEL_STREAM(128, 10, 8); break;
      default: return KVSEL_ERR_UNSUPPORTED;
    }
  } else {
    switch (nq) {
      case 1: KVSEL_STREAM(64, 1, 4); break;
      case 2: KVSEL_STREAM(64, 2, 4); break;
      case 4: KVSEL_STREAM(64, 4, 4); break;
      case 8: KVSEL_STREAM(64, 8, 4); break;
      case 10: KVSEL_STREAM(64, 10, 8); break;
      default: return KVSEL_ERR_UNSUPPORTED;
    }
  }
#undef KVSEL_STREAM
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
