// Window tiering (kvsel_route_tiers) for gfx950.
//
// QEvict ("Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding"), Sections 4.1-4.3: the cache is cut into
// contiguous windows, each window is scored by its accumulated attention,
// and windows are routed by rank into a full-precision tier, a recoverable
// low-bit tier and an evicted tier; low-bit windows are promoted back by
// dequantisation.  The low-bit code here is asymmetric int4 with one
// (lo, scale) pair per channel of a window; its exact rule is in kvsel.h.
//
// Kernels:
//   tier_rank_kernel     one workgroup per (batch, KV head): window sums in a
//                        fixed reduction order, exact rank by a bitonic sort,
//                        tier id, and each window's slot inside its tier
//   tier_move_kernel     one workgroup per window: full tier -> 16 B/lane row
//                        copy; int4 tier -> LDS-staged per-channel min/max,
//                        codes, nibble packing
//   tier_promote_kernel  one workgroup per promoted window: dequantise to bf16
#include <math.h>

#include "common.h"

namespace kvsel {
namespace {

constexpr int kWin = 64;
constexpr int kRankThreads = 1024;

__device__ __forceinline__ uint32_t block_excl_scan_1024(uint32_t v, uint32_t* total,
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
    uint32_t w = lane < 16 ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t t = __shfl_up(w, off);
      if (lane >= off) w += t;
    }
    if (lane < 16) wsum[lane] = w;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[wave - 1] : 0u;
  *total = wsum[15];
  __syncthreads();
  return before + incl - v;
}

// nwin <= 4096 windows per head.  Window sums in a fixed order, then the
// windows sorted by (sum desc, index asc) with a bitonic sort of unique 64-bit
// keys: a window's rank is its sorted position.
__global__ void __launch_bounds__(kRankThreads) tier_rank_kernel(
    const float* __restrict__ scores, int8_t* __restrict__ tier, int32_t* __restrict__ rank,
    int32_t* __restrict__ slot, int S, int nwin, int n_full, int n_quant) {
  __shared__ uint64_t key[4096];
  __shared__ int32_t rk[4096];
  __shared__ uint32_t wsum[16];
  const int head = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* s = scores + (size_t)head * S;
  int n2 = 1;
  while (n2 < nwin) n2 <<= 1;
  // Window sums: one wave per window, lane l adds tokens l; tree in fixed
  // order.  A wave takes its windows j, j + NWV, ... kSumBatch at a time, all
  // of a batch's loads issued before the first sum.
  constexpr int NWV = kRankThreads / 64, kSumBatch = 8;
  for (int j0 = wave; j0 < nwin; j0 += NWV * kSumBatch) {
    float x[kSumBatch];
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b)
      x[b] = s[(size_t)min(j0 + b * NWV, nwin - 1) * kWin + lane];
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) x[b] += __shfl_xor(x[b], off);
      if (lane == 0 && j0 + b * NWV < nwin) key[j0 + b * NWV] = desc_key(x[b], j0 + b * NWV);
    }
  }
  for (int j = nwin + tid; j < n2; j += kRankThreads) key[j] = ~0ull;
  __syncthreads();
  sort_keys<kRankThreads>(key, n2);
  for (int r = tid; r < nwin; r += kRankThreads) rk[(uint32_t)key[r]] = r;
  __syncthreads();
  uint32_t cf = 0u, cq = 0u;
  for (int base = 0; base < nwin; base += kRankThreads) {
    const int j = base + tid;
    int t = 2;
    if (j < nwin) {
      const int r = rk[j];
      t = r < n_full ? 0 : (r < n_full + n_quant ? 1 : 2);
      rank[(size_t)head * nwin + j] = r;
      tier[(size_t)head * nwin + j] = (int8_t)t;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan_1024(((uint32_t)(t == 0) << 16) | (uint32_t)(t == 1), &tot,
                                             wsum);
    if (j < nwin)
      slot[(size_t)head * nwin + j] = t == 0 ? (int)(cf + (ex >> 16))
                                             : (t == 1 ? (int)(cq + (ex & 0xffffu)) : -1);
    cf += tot >> 16;
    cq += tot & 0xffffu;
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One workgroup per window.  Full tier: 16-byte row copy.  int4 tier: thread
// (tensor, 8-channel octet, token group) loads 8 tokens x 8 channels with
// 16-byte loads, keeps them in registers, reduces per-channel min/max through
// LDS, then writes its packed codes (4 bytes per token).
template <int D>
__global__ void __launch_bounds__(256) tier_move_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int8_t* __restrict__ tier, const int32_t* __restrict__ slot,
    uint16_t* __restrict__ k_full, uint16_t* __restrict__ v_full, uint8_t* __restrict__ k_codes,
    uint8_t* __restrict__ v_codes, float* __restrict__ k_meta, float* __restrict__ v_meta, int S,
    int nwin, int n_full, int n_quant) {
#pragma clang fp contract(off)
  constexpr int VPW = kWin * D * 2 / 16;       // 16-byte vectors per window per tensor
  constexpr int OCT = D / 8;                   // 8-channel octets per token
  constexpr int TG = 256 / (2 * OCT);          // token groups (8 for D=128, 16 for D=64)
  constexpr int TPT = kWin / TG;               // tokens per thread (8 or 4)
  __shared__ float red_lo[TG][2][D], red_hi[TG][2][D];
  __shared__ float lo_s[2][D], sc_s[2][D];
  const int j = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int t = tier[(size_t)head * nwin + j];
  if (t == 2) return;
  const int sl = slot[(size_t)head * nwin + j];
  // Ranks form a permutation for finite scores, so slots stay below the tier
  // capacity; the guard keeps malformed scores from writing out of bounds.
  if (sl < 0 || sl >= (t == 0 ? n_full : n_quant)) return;
  const size_t src = ((size_t)head * S + (size_t)j * kWin) * D;
  if (t == 0) {
    const size_t dst = ((size_t)head * n_full * kWin + (size_t)sl * kWin) * D;
    const u32x4_t* ks = (const u32x4_t*)(k + src);
    const u32x4_t* vs = (const u32x4_t*)(v + src);
    u32x4_t* kd = (u32x4_t*)(k_full + dst);
    u32x4_t* vd = (u32x4_t*)(v_full + dst);
    for (int i = tid; i < VPW; i += 256) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
    return;
  }
  // int4 tier.
  const int tn = tid / (OCT * TG);             // 0 = K, 1 = V
  const int rem = tid - tn * (OCT * TG);
  const int oct = rem % OCT, tg = rem / OCT;
  const uint16_t* x = (tn == 0 ? k : v) + src;
  float val[TPT][8];
#pragma unroll
  for (int r = 0; r < TPT; ++r) {
    const u32x4_t w = *(const u32x4_t*)(x + (size_t)(tg * TPT + r) * D + oct * 8);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      val[r][2 * h] = __uint_as_float(w[h] << 16);
      val[r][2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
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
  // Per (tensor, channel): reduce the token groups, form (lo, scale).
  for (int id = tid; id < 2 * D; id += 256) {
    const int tt = id / D, ch = id - tt * D;
    float lo = red_lo[0][tt][ch], hi = red_hi[0][tt][ch];
    for (int g2 = 1; g2 < TG; ++g2) {
      lo = fminf(lo, red_lo[g2][tt][ch]);
      hi = fmaxf(hi, red_hi[g2][tt][ch]);
    }
    const float sc = (hi - lo) / 15.0f;
    lo_s[tt][ch] = lo;
    sc_s[tt][ch] = sc;
    float* meta = tt == 0 ? k_meta : v_meta;
    const size_t mo = (((size_t)head * n_quant + sl) * D + ch) * 2;
    meta[mo] = lo;
    meta[mo + 1] = sc;
  }
  __syncthreads();
  // Codes for this thread's 8 channels of each of its tokens: 4 packed bytes.
  float lo8[8], sc8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    lo8[c] = lo_s[tn][oct * 8 + c];
    sc8[c] = sc_s[tn][oct * 8 + c];
  }
  constexpr int BPT = D / 2;  // packed bytes per token
  uint8_t* codes = (tn == 0 ? k_codes : v_codes) + ((size_t)head * n_quant + sl) * kWin * BPT;
#pragma unroll
  for (int r = 0; r < TPT; ++r) {
    uint32_t word = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t code = 0u;
      if (sc8[c] != 0.f) {
        float qf = rintf((val[r][c] - lo8[c]) / sc8[c]);
        qf = fminf(fmaxf(qf, 0.f), 15.f);
        code = (uint32_t)qf;
      }
      word |= code << (4 * c);
    }
    *(uint32_t*)(codes + (size_t)(tg * TPT + r) * BPT + oct * 4) = word;
  }
}

template <int D>
__global__ void __launch_bounds__(256) tier_promote_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ k_meta, const float* __restrict__ v_meta,
    const int32_t* __restrict__ promote, uint16_t* __restrict__ k_prom,
    uint16_t* __restrict__ v_prom, int n_quant, int n_promote) {
  // The dequantised value is defined with two roundings (product, then sum):
  // forbid fusing them into one multiply-add.
#pragma clang fp contract(off)
  constexpr int BPT = D / 2;
  const int pi = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int sl = promote[(size_t)head * n_promote + pi];
  const bool ok = sl >= 0 && sl < n_quant;
  // Each thread writes 8 bf16 (16 bytes) = 8 channels of one token.
  for (int id = tid; id < 2 * kWin * (D / 8); id += 256) {
    const int tn = id / (kWin * (D / 8));
    const int rem = id - tn * (kWin * (D / 8));
    const int r = rem / (D / 8), c8 = (rem - r * (D / 8)) * 8;
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (ok) {
      const uint8_t* codes = (tn == 0 ? k_codes : v_codes) +
                             (((size_t)head * n_quant + sl) * kWin + r) * BPT + c8 / 2;
      const float* meta = (tn == 0 ? k_meta : v_meta) + (((size_t)head * n_quant + sl) * D) * 2;
      const uint32_t packed = *(const uint32_t*)codes;  // 8 codes
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = c8 + e;
        const uint32_t code = (packed >> (4 * e)) & 0xfu;
        const float lo = meta[2 * ch], sc = meta[2 * ch + 1];
        const float prod = (float)code * sc;
        const float x = lo + prod;
        out[e >> 1] |= (uint32_t)f32_to_bf16_rne(x) << (16 * (e & 1));
      }
    }
    uint16_t* dst = (tn == 0 ? k_prom : v_prom) +
                    (((size_t)head * n_promote + pi) * kWin + r) * D + c8;
    *(u32x4_t*)dst = u32x4_t{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace

bool plan_tiers(const kvsel_tier_desc& d, TierPlan* p) {
  p->nheads = d.batch * d.n_kv_heads;
  p->nwin = d.seq_len / d.win;
  p->off_slot = 0;
  p->total = align256((size_t)p->nheads * p->nwin * sizeof(int32_t));
  return true;
}

kvsel_status launch_tiers(const kvsel_tier_desc& d, const TierPlan& p, const float* scores,
                          const void* k, const void* v, int8_t* tier, int32_t* rank,
                          void* k_full, void* v_full, uint8_t* k_codes, uint8_t* v_codes,
                          float* k_meta, float* v_meta, const int32_t* promote, int n_promote,
                          void* k_prom, void* v_prom, char* ws, hipStream_t stream) {
  int32_t* slot = (int32_t*)(ws + p.off_slot);
  KVSEL_LAUNCH("tier_rank_kernel", tier_rank_kernel, dim3(p.nheads), dim3(kRankThreads), 0, stream, scores,
                     tier, rank, slot, d.seq_len, p.nwin, d.n_full, d.n_quant);
  const dim3 g(p.nwin, p.nheads);
  if (d.head_dim == 128) {
    KVSEL_LAUNCH("tier_move_kernel", tier_move_kernel<128>, g, dim3(256), 0, stream, (const uint16_t*)k,
                       (const uint16_t*)v, tier, slot, (uint16_t*)k_full, (uint16_t*)v_full,
                       k_codes, v_codes, k_meta, v_meta, d.seq_len, p.nwin, d.n_full, d.n_quant);
    if (n_promote > 0)
      KVSEL_LAUNCH("tier_promote_kernel", tier_promote_kernel<128>, dim3(n_promote, p.nheads), dim3(256), 0,
                         stream, k_codes, v_codes, k_meta, v_meta, promote, (uint16_t*)k_prom,
                         (uint16_t*)v_prom, d.n_quant, n_promote);
  } else {
    KVSEL_LAUNCH("tier_move_kernel", tier_move_kernel<64>, g, dim3(256), 0, stream, (const uint16_t*)k,
                       (const uint16_t*)v, tier, slot, (uint16_t*)k_full, (uint16_t*)v_full,
                       k_codes, v_codes, k_meta, v_meta, d.seq_len, p.nwin, d.n_full, d.n_quant);
    if (n_promote > 0)
      KVSEL_LAUNCH("tier_promote_kernel", tier_promote_kernel<64>, dim3(n_promote, p.nheads), dim3(256), 0,
                         stream, k_codes, v_codes, k_meta, v_meta, promote, (uint16_t*)k_prom,
                         (uint16_t*)v_prom, d.n_quant, n_promote);
  }
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
