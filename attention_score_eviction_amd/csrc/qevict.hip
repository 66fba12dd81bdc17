// Repeated recoverable routing (kvsel_qevict_step) for gfx950.
//
// QEvict ("Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding"), Sections 4.1-4.3 and Appendix A, run every Omega
// decode tokens, with the persistent quantised backing store of Section 1.
// Between the protected sink and recent regions the cache is cut into
// 64-token windows.  One routing step, per (sequence, KV head):
//   * accumulate each window's attention mass of this step into its score;
//   * rank the windows that are not evicted (score desc, index asc): the first
//     n_full stay / become full precision, the next n_quant quantised, the
//     rest are evicted for good;
//   * a window leaving the full tier for the quantised tier is quantised from
//     its cache rows at its first demotion only; later demotions reuse the
//     backing-store entry, so transitions do not accumulate error;
//   * a window promoted back to the full tier gets its cache rows rewritten
//     with the dequantised values (residency is restored, not the original
//     values).
// The low-bit code is asymmetric INT2 (the default tier) or INT4, one
// (lo, scale) pair per channel of a window, K and V separately.
//
// Kernels:
//   qe_rank_kernel  one workgroup per (sequence, KV head): window sums in a
//                   fixed reduction order, accumulation, exact rank among the
//                   live windows by a bitonic sort, new tier, and the data
//                   action of each window (none / first demotion / promotion)
//   qe_move_kernel  one workgroup per window with an action: quantise the
//                   window into its backing-store slot, or dequantise the slot
//                   into the cache rows
#include <math.h>

#include "common.h"

namespace kvsel {
namespace {

constexpr int kQeWin = 64;
constexpr int kQeRankThreads = 1024;
constexpr int kQeMaxWindows = 4096;
constexpr int8_t kActNone = 0, kActQuant = 1, kActPromote = 2;

__global__ void __launch_bounds__(kQeRankThreads) qe_rank_kernel(
    const float* __restrict__ scores, float* __restrict__ w_acc, int8_t* __restrict__ tier,
    uint8_t* __restrict__ has_codes, int8_t* __restrict__ act, int S, int n_sink, int nwin,
    int max_windows, int n_full, int n_quant) {
  __shared__ uint64_t key[kQeMaxWindows];   // (live score desc, index asc); evicted last
  __shared__ int32_t rk[kQeMaxWindows];
  const int head = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* s = scores + (size_t)head * S + n_sink;
  const size_t so = (size_t)head * max_windows;
  int n2 = 1;
  while (n2 < nwin) n2 <<= 1;
  // Window sums: one wave per window, lane l adds token l, a fixed butterfly.
  // A wave takes its windows j, j + NWV, ... kSumBatch at a time, with the
  // scores, accumulated sums and tiers of the batch all loaded before the
  // first sum (one memory latency per batch, not per window).
  constexpr int NWV = kQeRankThreads / 64, kSumBatch = 8;
  for (int j0 = wave; j0 < nwin; j0 += NWV * kSumBatch) {
    float x[kSumBatch], old[kSumBatch];
    int8_t t[kSumBatch];
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b) {
      const int j = min(j0 + b * NWV, nwin - 1);
      x[b] = s[(size_t)j * kQeWin + lane];
      old[b] = w_acc[so + j];
      t[b] = tier[so + j];
    }
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b) {
      const int j = j0 + b * NWV;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) x[b] += __shfl_xor(x[b], off);
      if (lane == 0 && j < nwin) {
        const float acc = old[b] + x[b];
        w_acc[so + j] = acc;
        // an evicted window sorts after every live one (its key's top bits
        // are all ones, above -inf's)
        key[j] = t[b] == 2 ? (0xffffffff00000000ull | (uint32_t)j) : desc_key(acc, j);
      }
    }
  }
  for (int j = nwin + tid; j < n2; j += kQeRankThreads) key[j] = ~0ull;
  __syncthreads();
  sort_keys<kQeRankThreads>(key, n2);
  for (int r = tid; r < nwin; r += kQeRankThreads) rk[(uint32_t)key[r]] = r;
  __syncthreads();
  // Live windows occupy the first sorted positions, so a live window's sorted
  // position is its rank among the live windows.
  for (int j = tid; j < nwin; j += kQeRankThreads) {
    const int8_t told = tier[so + j];
    if (told == 2) {
      act[so + j] = kActNone;
      continue;
    }
    const int r = rk[j];
    const int8_t tnew = r < n_full ? 0 : (r < n_full + n_quant ? 1 : 2);
    int8_t a = kActNone;
    if (told == 0 && tnew == 1 && has_codes[so + j] == 0) {
      a = kActQuant;
      has_codes[so + j] = 1;
    } else if (told == 1 && tnew == 0) {
      a = kActPromote;
    }
    act[so + j] = a;
    tier[so + j] = tnew;
  }
}

__device__ __forceinline__ uint16_t qe_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One workgroup per window.  Thread (tensor, 8-channel octet, token group)
// holds 8 channels of TPT tokens.  Quantise: per-channel min/max reduced
// through LDS, IEEE division, rint, packing (8 codes = BITS bytes per token
// octet).  Promote: dequantise 8 channels of each of its tokens, bf16 RNE,
// one 16-byte store per token.
template <int D, int BITS>
__global__ void __launch_bounds__(256) qe_move_kernel(
    uint16_t* __restrict__ k, uint16_t* __restrict__ v, const int8_t* __restrict__ act,
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, float* __restrict__ k_meta,
    float* __restrict__ v_meta, int cap, int n_sink, int max_windows) {
  // The quantiser divides and the dequantiser multiplies then adds, each
  // rounded once: no fused multiply-add.
#pragma clang fp contract(off)
  constexpr int OCT = D / 8;                   // 8-channel octets per token
  constexpr int TG = 256 / (2 * OCT);          // token groups (8 for D=128, 16 for D=64)
  constexpr int TPT = kQeWin / TG;             // tokens per thread (8 or 4)
  constexpr int BPT = D * BITS / 8;            // packed bytes per token
  constexpr float kLevels = (float)((1 << BITS) - 1);
  __shared__ float red_lo[TG][2][D], red_hi[TG][2][D];
  __shared__ float lo_s[2][D], sc_s[2][D];
  const int j = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const size_t so = (size_t)head * max_windows + j;
  const int a = act[so];
  if (a == kActNone) return;
  const int tn = tid / (OCT * TG);             // 0 = K, 1 = V
  const int rem = tid - tn * (OCT * TG);
  const int oct = rem % OCT, tg = rem / OCT;
  uint16_t* x = (tn == 0 ? k : v) + ((size_t)head * cap + n_sink + (size_t)j * kQeWin) * D;
  uint8_t* codes = (tn == 0 ? k_codes : v_codes) + so * kQeWin * BPT;
  float* meta = (tn == 0 ? k_meta : v_meta) + so * D * 2;

  if (a == kActPromote) {
    float lo8[8], sc8[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lo8[c] = meta[(oct * 8 + c) * 2];
      sc8[c] = meta[(oct * 8 + c) * 2 + 1];
    }
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int tok = tg * TPT + r;
      uint32_t packed;
      if constexpr (BITS == 4) packed = *(const uint32_t*)(codes + (size_t)tok * BPT + oct * 4);
      else packed = *(const uint16_t*)(codes + (size_t)tok * BPT + oct * 2);
      uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t code = (packed >> (BITS * c)) & ((1u << BITS) - 1u);
        const float prod = (float)code * sc8[c];
        const float y = lo8[c] + prod;
        out[c >> 1] |= (uint32_t)qe_bf16_rne(y) << (16 * (c & 1));
      }
      *(u32x4_t*)(x + (size_t)tok * D + oct * 8) = u32x4_t{out[0], out[1], out[2], out[3]};
    }
    return;
  }

  // First demotion: quantise the window's rows into the backing store.
  float val[TPT][8];
#pragma unroll
  for (int r = 0; r < TPT; ++r) {
    const u32x4_t wv = *(const u32x4_t*)(x + (size_t)(tg * TPT + r) * D + oct * 8);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      val[r][2 * h] = __uint_as_float(wv[h] << 16);
      val[r][2 * h + 1] = __uint_as_float(wv[h] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float lo = val[0][c], hi = val[0][c];
#pragma unroll
    for (int r = 1; r < TPT; ++r) {
      lo = fminf(lo, val[r][c]);
      hi = fmaxf(hi, val[r][c]);
    }
    red_lo[tg][tn][oct * 8 + c] = lo;
    red_hi[tg][tn][oct * 8 + c] = hi;
  }
  __syncthreads();
  for (int id = tid; id < 2 * D; id += 256) {
    const int tt = id / D, ch = id - tt * D;
    float lo = red_lo[0][tt][ch], hi = red_hi[0][tt][ch];
    for (int g2 = 1; g2 < TG; ++g2) {
      lo = fminf(lo, red_lo[g2][tt][ch]);
      hi = fmaxf(hi, red_hi[g2][tt][ch]);
    }
    const float sc = (hi - lo) / kLevels;
    lo_s[tt][ch] = lo;
    sc_s[tt][ch] = sc;
    float* mt = (tt == 0 ? k_meta : v_meta) + (so * D + ch) * 2;
    mt[0] = lo;
    mt[1] = sc;
  }
  __syncthreads();
  float lo8[8], sc8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    lo8[c] = lo_s[tn][oct * 8 + c];
    sc8[c] = sc_s[tn][oct * 8 + c];
  }
#pragma unroll
  for (int r = 0; r < TPT; ++r) {
    uint32_t word = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t code = 0u;
      if (sc8[c] != 0.f) {
        float qf = rintf((val[r][c] - lo8[c]) / sc8[c]);
        qf = fminf(fmaxf(qf, 0.f), kLevels);
        code = (uint32_t)qf;
      }
      word |= code << (BITS * c);
    }
    const int tok = tg * TPT + r;
    if constexpr (BITS == 4) *(uint32_t*)(codes + (size_t)tok * BPT + oct * 4) = word;
    else *(uint16_t*)(codes + (size_t)tok * BPT + oct * 2) = (uint16_t)word;
  }
}

template <int D>
void launch_qe_move(const kvsel_qevict_desc& d, dim3 g, void* k, void* v, const int8_t* act,
                    uint8_t* k_codes, uint8_t* v_codes, float* k_meta, float* v_meta,
                    hipStream_t stream) {
  if (d.bits == 2)
    KVSEL_LAUNCH("qe_move_kernel", (qe_move_kernel<D, 2>), g, dim3(256), 0, stream, (uint16_t*)k,
                       (uint16_t*)v, act, k_codes, v_codes, k_meta, v_meta, d.capacity,
                       d.n_sink, d.max_windows);
  else
    KVSEL_LAUNCH("qe_move_kernel", (qe_move_kernel<D, 4>), g, dim3(256), 0, stream, (uint16_t*)k,
                       (uint16_t*)v, act, k_codes, v_codes, k_meta, v_meta, d.capacity,
                       d.n_sink, d.max_windows);
}

}  // namespace

int qevict_windows(const kvsel_qevict_desc& d) {
  const int hist = d.seq_len - d.n_sink - d.n_recent;
  return hist > 0 ? hist / kQeWin : 0;
}

size_t qevict_workspace(const kvsel_qevict_desc& d) {
  return align256((size_t)d.batch * d.n_kv_heads * d.max_windows);
}

kvsel_status launch_qevict(const kvsel_qevict_desc& d, const float* scores, float* w_acc,
                           int8_t* tier, uint8_t* has_codes, void* k, void* v, uint8_t* k_codes,
                           uint8_t* v_codes, float* k_meta, float* v_meta, char* ws,
                           hipStream_t stream) {
  const int nheads = d.batch * d.n_kv_heads;
  const int nwin = qevict_windows(d);
  if (nwin == 0) return KVSEL_OK;
  int8_t* act = (int8_t*)ws;
  KVSEL_LAUNCH("qe_rank_kernel", qe_rank_kernel, dim3(nheads), dim3(kQeRankThreads), 0, stream, scores,
                     w_acc, tier, has_codes, act, d.seq_len, d.n_sink, nwin, d.max_windows,
                     d.n_full, d.n_quant);
  const dim3 g(nwin, nheads);
  if (d.head_dim == 128)
    launch_qe_move<128>(d, g, k, v, act, k_codes, v_codes, k_meta, v_meta, stream);
  else
    launch_qe_move<64>(d, g, k, v, act, k_codes, v_codes, k_meta, v_meta, stream);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
