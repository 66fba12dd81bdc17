// Exact top-B selection with the mandatory set (kvsel_select,
// kvsel_select_adaptive) for gfx950.
//
// TideKV ("Delayed KV Eviction via Layer-Wise Chunked Prefill ..."),
// Section 4.2, Eq. (8): R = Top_k{p_i : i not mandatory} U mandatory.
// TideKV keeps the top-k in a streaming heap inside pass 2 (Algorithm 2);
// here the per-key scores are already a compact fp32 vector per KV head (a
// few MiB, resident in the last-level cache), so the k-th largest value is
// found exactly by a three-digit radix select over the fp32 bit patterns.
// Scores are >= 0, so the sign bit is always clear and bit order equals value
// order; the digits are bits 30..20 (exponent and three mantissa bits, an
// eighth of an octave per bin), 19..10 and 9..0.  Ties at the threshold keep
// the lowest positions.  The retained positions are emitted in ascending
// order with a block-wide prefix count.
//
// Short rows: one workgroup per (batch, KV head), the row held in registers,
// histograms in LDS.  Long rows and head groups: the sliced kernels below.
#include "common.h"
#include "select_util.h"

namespace kvsel {
namespace {

constexpr int kSelThreads = 1024;

// Each thread takes 16 consecutive scores per batch as four 16-byte loads,
// so a sweep keeps many bytes in flight per CU.  Elements outside [lo, hi)
// come back invalid.  The four loads are unconditional and independent: a
// vector that is not wholly inside [lo, hi) loads from the nearest one that
// is (same alignment), and only its valid elements, if any, are reloaded one
// by one.  (With a vector/scalar choice per load the compiler waits for each
// vector load before issuing the next: four memory latencies in a row.)
constexpr int kPerThread = 16;

__device__ __forceinline__ uint32_t load16(const uint32_t* row, int p0, int lo, int hi,
                                           uint32_t (&x)[kPerThread]) {
  // Starts of the vectors wholly inside [lo, hi) congruent to p0 mod 4.
  const int f_lo = lo + ((p0 - lo) & 3);
  const int f_hi = (hi - 4) - ((hi - 4 - p0) & 3);
  uint32_t valid = 0u, fix = 0u;
  if (f_lo <= f_hi) {
    u32x4_t w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int pc = min(max(p0 + 4 * v, f_lo), f_hi);
      w[v] = *(const u32x4_t*)(row + pc);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = p0 + 4 * v;
      const bool same = p >= f_lo && p <= f_hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = p + e;
        const bool ok = i >= lo && i < hi;
        valid |= (uint32_t)ok << (4 * v + e);
        fix |= (uint32_t)(ok && !same) << (4 * v + e);
        x[4 * v + e] = (ok && same) ? w[v][e] : 0u;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = p0 + e;
      const bool ok = i >= lo && i < hi;
      valid |= (uint32_t)ok << e;
      fix |= (uint32_t)ok << e;
      x[e] = 0u;
    }
  }
  if (fix) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if ((fix >> e) & 1u) x[e] = row[p0 + e];
  }
  return valid;
}

// Heads of one selection group the single-workgroup kernel takes.
constexpr int kMaxWgHeads = 64;

// Single-workgroup select for one selection group: hg consecutive KV-head
// rows (hg = 1: a per-head budget; hg = Hkv: the head-adaptive budget of one
// sequence).  Each row's candidates are cut into nsl slices of 16 scores
// (from a 16-byte aligned start at or below lo); slice j of the group is row
// j / nsl, slice j % nsl.  Batch b is slices [b*NT, (b+1)*NT), one per
// thread, so thread order within a batch is (head, position) order.  The
// first NB batches stay in registers for the whole kernel; later ones (only
// for rows longer than the sliced kernels take) are reloaded per pass.
//
// GATHER (kvsel_select_compact, per-head groups, n_keep <= kMaxFusedKeep):
// `reps` workgroups per group each run the same selection (it is
// deterministic), keep the retained positions in LDS, and copy their share
// of the retained K/V rows; replica 0 also writes the index row.  The short
// rows this serves leave most CUs idle, so the repeated selection costs
// nothing extra and the separate gather launch disappears.
constexpr int kMaxFusedKeep = 4096;

struct GatherArgs {
  const u32x4_t* k;   // [groups][S][vpr]
  const u32x4_t* v;   // nullable
  u32x4_t* ko;        // [groups][n_keep][vpr]
  u32x4_t* vo;
  int vpr;            // 16-byte vectors per row
  int reps;           // workgroups per group
};

template <int NT, int NB, bool GATHER>
__global__ void __launch_bounds__(NT) select_kernel(const float* __restrict__ pooled,
                                                    int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ head_off, int S,
                                                    int lo, int hi, int budget, int n_sink,
                                                    int W, int n_keep, int hg, int nsl,
                                                    GatherArgs ga) {
  // One histogram per digit, all cleared up front: a round is then one
  // barrier after its counts and one after the digit search.
  __shared__ __attribute__((aligned(16))) uint32_t hist[2048 + 1024 + 1024];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t kept[kMaxWgHeads];
  __shared__ int32_t sidx[GATHER ? kMaxFusedKeep : 1];   // retained positions, in order
  const int grp = GATHER ? (int)blockIdx.x / ga.reps : (int)blockIdx.x, tid = threadIdx.x;
  const int rep = GATHER ? (int)blockIdx.x - grp * ga.reps : 0;
  const bool writer = rep == 0;   // the replica that writes the index row
  const int seg = n_sink + W;
  int32_t* out = idx + (size_t)grp * n_keep;
  const int nbatch = (hg * nsl + NT - 1) / NT;

  // Slice of batch b for this thread: its head, first position and scores.
  auto slice_load = [&](int bt, uint32_t (&x)[kPerThread], int& h, int& p0) -> uint32_t {
    const int j = bt * NT + tid;
    h = j / nsl;
    if (h >= hg) {
      h = hg - 1;
      p0 = hi;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) x[e] = 0u;
      return 0u;
    }
    const size_t row = (size_t)grp * hg + h;
    const int base0 = lo - ((lo + (int)((row * S) & 3u)) & 3);
    p0 = base0 + (j - h * nsl) * kPerThread;
    return load16((const uint32_t*)pooled + row * S, p0, lo, hi, x);
  };
  uint32_t xr[NB][kPerThread];
  uint32_t vr[NB];
  if (budget > 0) {
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      int h, p0;
      vr[bt] = slice_load(bt, xr[bt], h, p0);
    }
  }
  // Head and first position of this thread's slice in batch bt (recomputed
  // rather than kept: fewer live registers).
  auto slice_at = [&](int bt, int& h, int& p0) {
    const int j = bt * NT + tid;
    h = j / nsl;
    if (h >= hg) {
      h = hg - 1;
      p0 = hi;
      return;
    }
    const size_t row = (size_t)grp * hg + h;
    const int base0 = lo - ((lo + (int)((row * S) & 3u)) & 3);
    p0 = base0 + (j - h * nsl) * kPerThread;
  };
  // Visit every batch in order: the register-resident ones unrolled, the
  // rest reloaded.
  auto for_batches = [&](auto&& fn) {
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      if (bt < nbatch) {
        int h, p0;
        slice_at(bt, h, p0);
        fn(xr[bt], vr[bt], h, p0);
      }
    }
    for (int bt = NB; bt < nbatch; ++bt) {
      uint32_t x[kPerThread];
      int h, p0;
      const uint32_t v = slice_load(bt, x, h, p0);
      fn(x, v, h, p0);
    }
  };
  for (int i = tid; i < 2048 + 1024 + 1024; i += NT) hist[i] = 0u;
  for (int i = tid; i < hg; i += NT) kept[i] = 0u;
  __syncthreads();

  if (budget > 0) {
    // Radix select: digit r covers bits [shift, shift+nbits).
    uint32_t prefix = 0u, pmask = 0u, rem = (uint32_t)budget;
    for (int r = 0; r < 3; ++r) {
      const int shift = r == 0 ? 20 : (r == 1 ? 10 : 0);
      const int nb = r == 0 ? 2048 : 1024;
      uint32_t* hh = hist + (r == 0 ? 0 : (r == 1 ? 2048 : 3072));
      for_batches([&](const uint32_t (&x)[kPerThread], uint32_t valid, int, int) {
        uint32_t bin[kPerThread];
        uint32_t act = 0u;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          bin[e] = (x[e] >> shift) & (uint32_t)(nb - 1);
          act |= (uint32_t)(((valid >> e) & 1u) && (x[e] & pmask) == prefix) << e;
        }
        if (r == 0) {
          hist_add_runs(hh, bin, act);
        } else {
          // later digits count only the scores that share the prefix, a
          // few per thread: one masked atomic each
#pragma unroll
          for (int e = 0; e < kPerThread; ++e)
            if ((act >> e) & 1u) atomicAdd(&hh[bin[e]], 1u);
        }
      });
      __syncthreads();
      if (r == 0) block_find_digit<2048>(hh, rem, pick);
      else block_find_digit<1024>(hh, rem, pick);
      const uint32_t digit = pick[0];
      rem -= pick[1];
      prefix |= digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      // The whole boundary bin is kept: no need to resolve the lower bits.
      if (rem == pick[2]) break;
    }
    // Kept: (x & pmask) > prefix, and the first `rem` elements in (head,
    // position) order with (x & pmask) == prefix.  After three rounds pmask
    // covers every bit below the sign and prefix is the exact bit pattern of
    // the budget-th largest score.  Pick number `slot` of the group goes to
    // row h*(n_sink+W) + n_sink + slot: the rows of earlier heads' picks and
    // mandatory sets come before it.
    const uint32_t need_eq = rem;
    uint32_t cgt = 0u, ceq = 0u;
    for_batches([&](const uint32_t (&x)[kPerThread], uint32_t valid, int h, int p0) {
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
      const uint32_t ex = block_exclusive_scan<NT>((ngt << 16) | neq, &tot, wsum);
      const uint32_t gtb = cgt + (ex >> 16), eqb = ceq + (ex & 0xffffu);
      // Every score above the prefix is kept, and the first need_eq equal
      // ones of the group: eq_before of them lie in earlier threads, this
      // thread keeps its first `take`.  Both come from min() so that no
      // unsigned difference can wrap (the guarded form
      // `eqb < need_eq ? need_eq - eqb : 0` was compiled without its guard
      // by this toolchain, which misplaced every pick after a tie run).
      const uint32_t eq_before = min(eqb, need_eq);
      const uint32_t take = min(neq, need_eq - eq_before);
      uint32_t keep = gt;
      for (uint32_t i = 0, m = eq; i < take; ++i) {
        keep |= m & (0u - m);
        m &= m - 1u;
      }
      // The kept scores of this thread take consecutive slots from `slot`,
      // in position order.
      uint32_t slot = gtb + eq_before;
      int32_t* oh = out + h * seg + n_sink;
      uint32_t nw = 0u;
      while (keep) {
        const int e = __builtin_ctz(keep);
        keep &= keep - 1u;
        // slot < budget always holds for finite non-negative scores; the
        // guard keeps malformed input from writing outside this group.
        if (slot < (uint32_t)budget) {
          if (writer) oh[slot] = p0 + e;
          if constexpr (GATHER) sidx[h * seg + n_sink + slot] = p0 + e;
          ++nw;
        }
        ++slot;
      }
      if (hg > 1 && nw) atomicAdd(&kept[h], nw);
      cgt += tot >> 16;
      ceq += tot & 0xffffu;
    });
    // One head: its pick count is the number of slots filled.
    if (hg == 1 && tid == 0) kept[0] = min((uint32_t)budget, cgt + min(ceq, need_eq));
  }
  __syncthreads();
  // Mandatory rows and head offsets from the per-head pick counts.
  auto picks_before = [&](int h) -> uint32_t {
    uint32_t c = 0u;
    for (int k = 0; k < h; ++k) c += kept[k];
    return c;
  };
  if (head_off && writer)
    for (int h = tid; h <= hg; h += NT)
      head_off[(size_t)grp * (hg + 1) + h] = (int32_t)(h * seg + picks_before(h));
  for (int t = tid; t < hg * seg; t += NT) {
    const int h = t / seg, j = t - h * seg;
    const uint32_t start = h * seg + picks_before(h);
    const uint32_t row = j < n_sink ? start + j : start + n_sink + kept[h] + (j - n_sink);
    const int32_t pos = j < n_sink ? j : S - W + (j - n_sink);
    if (writer) out[row] = pos;
    if constexpr (GATHER) sidx[row] = pos;
  }
  if constexpr (GATHER) {
    // This replica's share of the retained rows (one KV head per group).
    __syncthreads();
    const int share = (n_keep + ga.reps - 1) / ga.reps;
    const int r0 = rep * share, r1 = min(n_keep, r0 + share);
    const int vpr = ga.vpr;
    for (int t = tid; t < (r1 - r0) * vpr; t += NT) {
      const int r = r0 + t / vpr, c = t - (t / vpr) * vpr;
      const int src = sidx[r];
      const bool ok = src >= 0 && src < S;
      const size_t so = ((size_t)grp * S + (ok ? src : 0)) * vpr + c;
      const size_t dst = ((size_t)grp * n_keep + r) * vpr + c;
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      const u32x4_t kx = ok ? ga.k[so] : zero;
      if (ga.v) {
        const u32x4_t vx = ok ? ga.v[so] : zero;
        ga.ko[dst] = kx;
        ga.vo[dst] = vx;
      } else {
        ga.ko[dst] = kx;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup select for long rows and for head-adaptive selection.
// A selection group is `hg` consecutive KV-head rows of one sequence (hg = 1:
// one row, the per-head budget of Eq. (8); hg = Hkv: the sequence-wide budget
// of TideKV Section 4.1's head-adaptive variant).  Each row's candidate range
// is cut into ns slices of kSlice scores (256 threads x 16); the group's
// slices are numbered head-major.  The kernels run in order:
//   sel_init     zero the group's two digit histograms
//   sel_hist     per slice: first-digit (bits 30..20) histogram -> global
//   sel_hist2    per slice: first digit d1 of the budget-th score; histogram
//                of the second digit (bits 19..10) of the scores in d1's bin
//   sel_cand     per slice: the 21-bit prefix of the budget-th score; count
//                the scores above it and compact the ones that share it
//   sel_resolve  per group: the last 10 bits over the compacted scores, the
//                tie cut (by head, then position), each slice's output
//                offset, the per-head offsets and the mandatory rows
//   sel_emit     per slice: ordered write of the kept positions
// Both wide digits are settled by every slice in parallel, so the single
// resolve workgroup only sees scores equal to the budget-th one in their
// bits 30..10 (a handful, unless values repeat).  A digit whose boundary bin is
// kept whole ends the search early.
// The rule every kernel applies in the end is one predicate per score:
// kept <=> key > prefix || (key == prefix && h*S + position <= cut), with
// key = bits & pmask and h the head's index inside its group.
//
// Output of a group: head h's rows start at h*(n_sink+W) + (picks of heads
// before h); they are its sinks, its picks in ascending position order and its
// observation window.  With hg = 1 this is the [sinks | picks | window] row.
// ---------------------------------------------------------------------------
constexpr int kSliceThreads = 256;
constexpr int kSlice = kSliceThreads * kPerThread;
constexpr int kD1Bits = 11, kD1Bins = 1 << kD1Bits, kD1Shift = 31 - kD1Bits;
constexpr int kD2Bits = 10, kD2Bins = 1 << kD2Bits, kD2Shift = kD1Shift - kD2Bits;
constexpr int kD3Bins = 1 << kD2Shift;

struct SelArgs {
  const float* pooled;
  int32_t* idx;        // [groups][n_keep]
  int32_t* head_off;   // [groups][hg+1] or null
  uint32_t* hist1;     // [groups][kD1Bins]
  uint32_t* hist2;     // [groups][kD2Bins]
  uint32_t* gtc;       // [groups][nst] scores kept outright (above the prefix)
  uint32_t* candc;     // [groups][nst] scores sharing the prefix (compacted)
  uint32_t* offs;      // [groups][nst] output offset (among picks) of each slice
  uint32_t* params;    // [groups][4] prefix, pmask, cut
  uint32_t* cval;      // [groups][nst][kSlice] compacted score bits
  int32_t* cidx;       // [groups][nst][kSlice] their keys h*S + position
  int S, lo, hi, budget, n_sink, W, n_keep, ns, hg, nst;
};

// Slice sg of group grp: its KV-head row and its slice number inside the row.
struct SliceAt {
  int h, row, sl;
};
__device__ __forceinline__ SliceAt slice_at(const SelArgs& a, int grp, int sg) {
  SliceAt r;
  r.h = sg / a.ns;
  r.sl = sg - r.h * a.ns;
  r.row = grp * a.hg + r.h;
  return r;
}

__device__ __forceinline__ int slice_base(const SelArgs& a, int row) {
  const int ofs = (int)(((size_t)row * a.S) & 3u);
  return a.lo - ((a.lo + ofs) & 3);
}

// The digits settled from the global histograms: prefix / pmask of the
// budget-th score over the first one or two digits, the rank still to place
// inside that prefix, and whether every score sharing it is kept.
struct Prefix {
  uint32_t prefix, pmask, rem;
  bool whole;
};

// hist1 / hist2 are LDS copies; hist2 is read only when the first digit's
// bin is not kept whole.  Every thread of the block must call.
template <int NT>
__device__ __forceinline__ Prefix settle_prefix(const uint32_t* hist1, const uint32_t* hist2,
                                                uint32_t budget, uint32_t* pick) {
  Prefix p;
  block_find_digit<kD1Bins>(hist1, budget, pick);
  p.rem = budget - pick[1];
  p.prefix = pick[0] << kD1Shift;
  p.pmask = (uint32_t)(kD1Bins - 1) << kD1Shift;
  p.whole = p.rem == pick[2];
  __syncthreads();
  if (!p.whole) {
    block_find_digit<kD2Bins>(hist2, p.rem, pick);
    p.rem -= pick[1];
    p.prefix |= pick[0] << kD2Shift;
    p.pmask |= (uint32_t)(kD2Bins - 1) << kD2Shift;
    p.whole = p.rem == pick[2];
    __syncthreads();
  }
  return p;
}

__global__ void __launch_bounds__(256) sel_init(SelArgs a) {
  const int grp = blockIdx.x, tid = threadIdx.x;
  uint32_t* h1 = a.hist1 + (size_t)grp * kD1Bins;
  uint32_t* h2 = a.hist2 + (size_t)grp * kD2Bins;
  for (int i = tid; i < kD1Bins; i += 256) h1[i] = 0u;
  for (int i = tid; i < kD2Bins; i += 256) h2[i] = 0u;
}

__global__ void __launch_bounds__(kSliceThreads) sel_hist(SelArgs a) {
  __shared__ uint32_t hist[kD1Bins];
  const int grp = blockIdx.y, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, blockIdx.x);
  for (int i = tid; i < kD1Bins; i += kSliceThreads) hist[i] = 0u;
  __syncthreads();
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  {
    uint32_t bin[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) bin[e] = (x[e] >> kD1Shift) & (uint32_t)(kD1Bins - 1);
    hist_add_runs(hist, bin, valid);
  }
  __syncthreads();
  uint32_t* g = a.hist1 + (size_t)grp * kD1Bins;
  for (int i = tid; i < kD1Bins; i += kSliceThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ void __launch_bounds__(kSliceThreads) sel_hist2(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kD1Bins];
  __shared__ uint32_t hist[kD2Bins];
  __shared__ uint32_t pick[3];
  const int grp = blockIdx.y, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, blockIdx.x);
  const uint32_t* g1 = a.hist1 + (size_t)grp * kD1Bins;
  for (int i = tid; i < kD1Bins; i += kSliceThreads) h1[i] = g1[i];
  for (int i = tid; i < kD2Bins; i += kSliceThreads) hist[i] = 0u;
  __syncthreads();
  block_find_digit<kD1Bins>(h1, (uint32_t)a.budget, pick);
  const uint32_t d1 = pick[0];
  if ((uint32_t)a.budget - pick[1] == pick[2]) return;   // d1's bin kept whole
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  uint32_t bin[kPerThread];
  uint32_t act = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    bin[e] = (x[e] >> kD2Shift) & (uint32_t)(kD2Bins - 1);
    act |= (uint32_t)(((valid >> e) & 1u) && ((x[e] >> kD1Shift) & (uint32_t)(kD1Bins - 1)) == d1)
           << e;
  }
  hist_add_runs(hist, bin, act);
  __syncthreads();
  uint32_t* g2 = a.hist2 + (size_t)grp * kD2Bins;
  for (int i = tid; i < kD2Bins; i += kSliceThreads)
    if (hist[i]) atomicAdd(&g2[i], hist[i]);
}

__global__ void __launch_bounds__(kSliceThreads) sel_cand(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kD1Bins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[kD2Bins];
  __shared__ uint32_t wsum[kSliceThreads / 64];
  __shared__ uint32_t pick[3];
  const int grp = blockIdx.y, sg = blockIdx.x, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, sg);
  const uint32_t* g1 = a.hist1 + (size_t)grp * kD1Bins;
  const uint32_t* g2 = a.hist2 + (size_t)grp * kD2Bins;
  for (int i = tid; i < kD1Bins; i += kSliceThreads) h1[i] = g1[i];
  for (int i = tid; i < kD2Bins; i += kSliceThreads) h2[i] = g2[i];
  __syncthreads();
  const Prefix pf = settle_prefix<kSliceThreads>(h1, h2, (uint32_t)a.budget, pick);
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  const int key0 = at.h * a.S + i0;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  uint32_t gt = 0u, in = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = (valid >> e) & 1u;
    const uint32_t key = x[e] & pf.pmask;
    gt += ok && (key > pf.prefix || (pf.whole && key == pf.prefix));
    in |= (uint32_t)(ok && !pf.whole && key == pf.prefix) << e;
  }
  uint32_t tot;
  uint32_t pos = block_exclusive_scan<kSliceThreads>((gt << 16) | __popc(in), &tot, wsum) & 0xffffu;
  const size_t cbase = ((size_t)grp * a.nst + sg) * kSlice;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((in >> e) & 1u) {
      a.cval[cbase + pos] = x[e];
      a.cidx[cbase + pos] = key0 + e;
      ++pos;
    }
  }
  if (tid == 0) {
    a.gtc[(size_t)grp * a.nst + sg] = tot >> 16;
    a.candc[(size_t)grp * a.nst + sg] = tot & 0xffffu;
  }
}

// Compacted scores held in LDS by sel_resolve (more spill to a slower path
// that reads them from global memory on every pass).
constexpr int kCandCap = 14336;

// Slice of flat candidate number k, given the exclusive prefix of the
// per-slice counts (cstart, ns entries, non-decreasing).
__device__ __forceinline__ int slice_of(const uint32_t* cstart, int ns, uint32_t k) {
  int lo = 0, hi = ns - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cstart[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kSelThreads) sel_resolve(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kD1Bins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[kD2Bins];
  __shared__ uint32_t selc[kMaxGroupSlices];
  __shared__ uint32_t cstart[kMaxGroupSlices];
  __shared__ uint32_t lval[kCandCap];
  __shared__ int32_t lidx[kCandCap];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t cut_s;
  const int grp = blockIdx.x, tid = threadIdx.x;
  const int ns = a.nst;   // slices of the whole group
  const uint32_t* g1 = a.hist1 + (size_t)grp * kD1Bins;
  const uint32_t* g2 = a.hist2 + (size_t)grp * kD2Bins;
  const uint32_t* cc = a.candc + (size_t)grp * ns;
  for (int i = tid; i < kD1Bins; i += kSelThreads) h1[i] = g1[i];
  for (int i = tid; i < kD2Bins; i += kSelThreads) h2[i] = g2[i];
  for (int i = tid; i < kMaxGroupSlices; i += kSelThreads) selc[i] = 0u;
  if (tid == 0) cut_s = 0x7fffffffu;
  // Flat numbering of the compacted scores (slice order = key order).
  uint32_t c0 = 0u, c1 = 0u;
  if (2 * tid < ns) c0 = cc[2 * tid];
  if (2 * tid + 1 < ns) c1 = cc[2 * tid + 1];
  uint32_t ncand;
  const uint32_t ex = block_exclusive_scan<kSelThreads>(c0 + c1, &ncand, wsum);
  if (2 * tid < ns) cstart[2 * tid] = ex;
  if (2 * tid + 1 < ns) cstart[2 * tid + 1] = ex + c0;
  __syncthreads();
  Prefix pf = settle_prefix<kSelThreads>(h1, h2, (uint32_t)a.budget, pick);
  uint32_t prefix = pf.prefix, pmask = pf.pmask, rem = pf.rem;
  const uint32_t* cv = a.cval + (size_t)grp * ns * kSlice;
  const int32_t* ci = a.cidx + (size_t)grp * ns * kSlice;
  const bool in_lds = ncand <= (uint32_t)kCandCap;
  if (!pf.whole) {
    // Gather the compacted scores into LDS with independent loads.
    if (in_lds) {
      for (uint32_t k = tid; k < ncand; k += kSelThreads) {
        const int sl = slice_of(cstart, ns, k);
        const size_t at = (size_t)sl * kSlice + (k - cstart[sl]);
        lval[k] = cv[at];
        lidx[k] = ci[at];
      }
      __syncthreads();
    }
    auto cand = [&](uint32_t k, uint32_t& v, int32_t& i) {
      if (in_lds) {
        v = lval[k];
        i = lidx[k];
      } else {
        const int sl = slice_of(cstart, ns, k);
        const size_t at = (size_t)sl * kSlice + (k - cstart[sl]);
        v = cv[at];
        i = ci[at];
      }
    };
    // Last digit (10 bits) over the compacted scores, which all share the
    // 21-bit prefix.  The histogram reuses h1.
    for (int i = tid; i < kD3Bins; i += kSelThreads) h1[i] = 0u;
    __syncthreads();
    for (uint32_t k0 = 0; k0 < ncand; k0 += kSelThreads) {
      const uint32_t k = k0 + tid;
      uint32_t x = 0u;
      int32_t key;
      if (k < ncand) cand(k, x, key);
      hist_add(h1, x & (uint32_t)(kD3Bins - 1), k < ncand);
    }
    __syncthreads();
    block_find_digit<kD3Bins>(h1, rem, pick);
    rem -= pick[1];
    prefix |= pick[0];
    pmask = 0xffffffffu;
    const bool whole3 = rem == pick[2];
    __syncthreads();
    // Tie cut: key (h*S + position) of the rem-th score equal to the prefix.
    // Each thread takes a contiguous run of candidates, so one scan orders
    // them.
    if (!whole3) {
      const uint32_t per = (ncand + kSelThreads - 1) / kSelThreads;
      const uint32_t k0 = tid * per, k1 = min(ncand, k0 + per);
      uint32_t neq = 0u;
      for (uint32_t k = k0; k < k1; ++k) {
        uint32_t x;
        int32_t key;
        cand(k, x, key);
        neq += x == prefix;
      }
      uint32_t tot;
      uint32_t seen = block_exclusive_scan<kSelThreads>(neq, &tot, wsum);
      if (seen < rem && rem <= seen + neq) {
        for (uint32_t k = k0; k < k1; ++k) {
          uint32_t x;
          int32_t key;
          cand(k, x, key);
          if (x == prefix && ++seen == rem) {
            cut_s = (uint32_t)key;
            break;
          }
        }
      }
      __syncthreads();
    }
    const uint32_t cut = cut_s;
    // Kept compacted scores per slice.
    for (uint32_t k0 = 0; k0 < ncand; k0 += kSelThreads) {
      const uint32_t k = k0 + tid;
      bool keep = false;
      int sl = 0;
      if (k < ncand) {
        uint32_t x;
        int32_t key;
        cand(k, x, key);
        keep = x > prefix || (x == prefix && (uint32_t)key <= cut);
        sl = slice_of(cstart, ns, k);
      }
      hist_add(selc, (uint32_t)sl, keep);
    }
  }
  __syncthreads();
  const uint32_t cut = cut_s;
  // Exclusive prefix over slices of (kept outright + kept compacted) counts.
  const uint32_t* gt = a.gtc + (size_t)grp * ns;
  uint32_t k0c = 0u, k1c = 0u;
  const int s0 = 2 * tid, s1 = 2 * tid + 1;
  if (s0 < ns) k0c = gt[s0] + selc[s0];
  if (s1 < ns) k1c = gt[s1] + selc[s1];
  uint32_t tot;
  const uint32_t exo = block_exclusive_scan<kSelThreads>(k0c + k1c, &tot, wsum);
  uint32_t* of = a.offs + (size_t)grp * ns;
  if (s0 < ns) of[s0] = exo;
  if (s1 < ns) of[s1] = exo + k0c;
  // Slice offsets also kept in LDS (cstart is free again) for the head offsets.
  if (s0 < ns) cstart[s0] = exo;
  if (s1 < ns) cstart[s1] = exo + k0c;
  if (tid == 0) {
    uint32_t* pr = a.params + (size_t)grp * 4;
    pr[0] = prefix;
    pr[1] = pmask;
    pr[2] = cut;
  }
  __syncthreads();
  // Head h's picks occupy [cstart[h*ns_row], next head's start) among the
  // group's picks; its rows start after the mandatory rows of earlier heads.
  const int seg = a.n_sink + a.W;
  auto picks_before = [&](int h) -> uint32_t {
    return h < a.hg ? min(cstart[h * a.ns], (uint32_t)a.budget) : (uint32_t)a.budget;
  };
  if (a.head_off)
    for (int h = tid; h <= a.hg; h += kSelThreads)
      a.head_off[(size_t)grp * (a.hg + 1) + h] = (int32_t)(h * seg + picks_before(h));
  int32_t* out = a.idx + (size_t)grp * a.n_keep;
  for (int t = tid; t < a.hg * seg; t += kSelThreads) {
    const int h = t / seg, j = t - h * seg;
    const uint32_t start = h * seg + picks_before(h);
    if (j < a.n_sink) {
      out[start + j] = j;
    } else {
      const int w = j - a.n_sink;
      out[start + a.n_sink + (picks_before(h + 1) - picks_before(h)) + w] = a.S - a.W + w;
    }
  }
}

__global__ void __launch_bounds__(kSliceThreads) sel_emit(SelArgs a) {
  __shared__ uint32_t wsum[kSliceThreads / 64];
  const int grp = blockIdx.y, sg = blockIdx.x, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, sg);
  const uint32_t* pr = a.params + (size_t)grp * 4;
  const uint32_t prefix = pr[0], pmask = pr[1], cut = pr[2];
  const uint32_t base_out = a.offs[(size_t)grp * a.nst + sg];
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  const uint32_t key0 = (uint32_t)(at.h * a.S + i0);
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  uint32_t keep = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t key = x[e] & pmask;
    const bool k = ((valid >> e) & 1u) &&
                   (key > prefix || (key == prefix && key0 + e <= cut));
    keep |= (uint32_t)k << e;
  }
  uint32_t tot;
  uint32_t pos = base_out + block_exclusive_scan<kSliceThreads>(__popc(keep), &tot, wsum);
  int32_t* out = a.idx + (size_t)grp * a.n_keep + at.h * (a.n_sink + a.W) + a.n_sink;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((keep >> e) & 1u) {
      // pos < budget for finite non-negative scores; guarded regardless.
      if (pos < (uint32_t)a.budget) out[pos] = i0 + e;
      ++pos;
    }
  }
}

// ---------------------------------------------------------------------------
// Layer-end selection of one KV-head row (hg = 1) straight from the raw
// scores, in three launches (plus the gather):
//
//   sel_pool_hist  the max filter, fused with the histogram of a 12-bit
//                  first digit (bits 30..19): each slice stages its raw
//                  scores with a halo, writes the pooled scores and adds its
//                  digits to the row's global histogram;
//   le_cand        every slice settles the first digit from that histogram,
//                  counts its scores above the digit's bin and compacts the
//                  ones inside it (about 1-2% of a row) in position order;
//   le_emit        every slice reads its row's compacted scores (into
//                  registers, or LDS when a slice holds more than its threads
//                  take) and settles the other 19 bits there (10 + 9, or a
//                  direct ranking when at most 64 candidates share the first
//                  22) and the tie cut -- the same result in every workgroup
//                  of the row, with no grid-wide step -- then takes its output
//                  offset from the per-slice counts and writes its picks;
//                  slice 0 also writes the sinks and the window.
//
// The kept set and its order are those of the generic sliced select above:
// the budget largest scores by (score desc, position asc), ascending.
// ---------------------------------------------------------------------------
constexpr int kLeD1Bits = 12, kLeD1Bins = 1 << kLeD1Bits, kLeD1Shift = 31 - kLeD1Bits;
constexpr int kLeD2Bits = 10, kLeD2Bins = 1 << kLeD2Bits, kLeD2Shift = kLeD1Shift - kLeD2Bits;
constexpr int kLeD3Bins = 1 << kLeD2Shift;
constexpr uint32_t kLeFullMask = 0x7fffffffu;
// Compacted scores a row may hold in le_emit's LDS (more are read from
// global memory on every pass instead: correct, slower), and the slices of
// a row whose counters le_emit keeps in LDS.
constexpr int kLeCandCap = 8192;
constexpr int kLeMaxSlices = 1024;

// Each slice stages its raw scores with a halo of h positions on either side
// (clipped to the candidate range [lo, hi)), writes the pooled scores of its
// positions, and adds their first digits to the row's global histogram
// (zeroed earlier on the stream).  The first and last slices of a row also
// write the zeros of the non-candidate positions [0, lo) and [hi, S).
constexpr int kMaxPoolHalo = 64;

// Histogram add of one element per lane, where lanes hold consecutive
// positions: a run of equal bins over consecutive lanes costs one atomic by
// its first lane (max-pooling repeats a local maximum over its neighbours).
// bin = ~0u marks an element that is not counted.
__device__ __forceinline__ void hist_add_lane_runs(uint32_t* hist, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  const uint32_t prev = (uint32_t)__builtin_amdgcn_ds_bpermute(((lane + 63) & 63) << 2, (int)bin);
  const bool start = lane == 0 || prev != bin;
  const unsigned long long starts = __ballot(start);
  if (!start || bin == ~0u) return;
  const unsigned long long above = lane == 63 ? 0ull : starts & (~0ull << (lane + 1));
  const int next = above ? __ffsll((long long)above) - 1 : 64;
  atomicAdd(&hist[bin], (uint32_t)(next - lane));
}

constexpr int kPoolThreads = 1024;

__global__ void __launch_bounds__(kPoolThreads) sel_pool_hist(SelArgs a, const float* raw,
                                                              float* pooled, int ph) {
  constexpr int NT = kPoolThreads, PER = kSlice / kPoolThreads;
  __shared__ uint32_t hist[kLeD1Bins];
  __shared__ float sv[kSlice + 2 * kMaxPoolHalo];
  const int grp = blockIdx.y, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, blockIdx.x);
  for (int i = tid; i < kLeD1Bins; i += NT) hist[i] = 0u;
  const size_t rbase = (size_t)at.row * a.S;
  const int base = slice_base(a, at.row) + at.sl * kSlice;
  {
    // Every load issued before the first is used: positions clamped into
    // the candidate range (always a valid address), out-of-range ones
    // replaced after the load.
    constexpr int NS = (kSlice + 2 * kMaxPoolHalo + NT - 1) / NT;
    float r[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int pos = base - ph + j * NT + tid;
      r[j] = raw[rbase + min(max(pos, a.lo), a.hi - 1)];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = j * NT + tid;
      const int pos = base - ph + i;
      if (i < kSlice + 2 * ph) sv[i] = (pos >= a.lo && pos < a.hi) ? r[j] : -INFINITY;
    }
  }
  __syncthreads();
  // Position base + j*NT + tid per step j: consecutive lanes read
  // consecutive LDS words and write consecutive pooled scores.
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int off = j * NT + tid;
    const int pos = base + off;
    const bool ok = pos >= a.lo && pos < a.hi;
    uint32_t bin = ~0u;
    if (ok) {
      const float* w = sv + off;   // positions pos - ph .. pos + ph
      float m = w[0];
      if (ph <= 3) {
#pragma unroll
        for (int t = 1; t <= 6; ++t)
          if (t <= 2 * ph) m = fmaxf(m, w[t]);
      } else {
        for (int t = 1; t <= 2 * ph; ++t) m = fmaxf(m, w[t]);
      }
      pooled[rbase + pos] = m;
      bin = (__float_as_uint(m) >> kLeD1Shift) & (uint32_t)(kLeD1Bins - 1);
    }
    hist_add_lane_runs(hist, bin);
  }
  if (at.sl == 0)
    for (int pos = tid; pos < a.lo; pos += NT) pooled[rbase + pos] = 0.f;
  if (at.sl == a.ns - 1)
    for (int pos = a.hi + tid; pos < a.S; pos += NT) pooled[rbase + pos] = 0.f;
  __syncthreads();
  uint32_t* g = a.hist1 + (size_t)grp * kLeD1Bins;
  for (int i = tid; i < kLeD1Bins; i += NT)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// For kvsel_select over long rows (scores already pooled): the first-digit
// histogram zeroed, then built from the pooled scores; le_cand and le_emit
// follow as in the layer-end path.
__global__ void __launch_bounds__(256) le_init(SelArgs a) {
  uint32_t* h1 = a.hist1 + (size_t)blockIdx.x * kLeD1Bins;
  uint32_t* h2 = a.hist1 + (size_t)gridDim.x * kLeD1Bins + (size_t)blockIdx.x * kLeD2Bins;
  for (int i = threadIdx.x; i < kLeD1Bins; i += 256) h1[i] = 0u;
  for (int i = threadIdx.x; i < kLeD2Bins; i += 256) h2[i] = 0u;
}

__global__ void __launch_bounds__(kSliceThreads) le_hist(SelArgs a) {
  __shared__ uint32_t hist[kLeD1Bins];
  const int grp = blockIdx.y, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, blockIdx.x);
  for (int i = tid; i < kLeD1Bins; i += kSliceThreads) hist[i] = 0u;
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  uint32_t bin[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) bin[e] = (x[e] >> kLeD1Shift) & (uint32_t)(kLeD1Bins - 1);
  __syncthreads();
  hist_add_runs(hist, bin, valid);
  __syncthreads();
  uint32_t* g = a.hist1 + (size_t)grp * kLeD1Bins;
  for (int i = tid; i < kLeD1Bins; i += kSliceThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ void __launch_bounds__(kSliceThreads) le_cand(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kLeD1Bins];
  __shared__ uint32_t wsum[kSliceThreads / 64];
  __shared__ uint32_t pick[3];
  const int grp = blockIdx.y, sg = blockIdx.x, tid = threadIdx.x;
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)grp * a.S;
  const int i0 = slice_base(a, grp) + sg * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  {
    constexpr int NV = kLeD1Bins / (4 * kSliceThreads);
    const u32x4_t* g1 = (const u32x4_t*)(a.hist1 + (size_t)grp * kLeD1Bins);
    u32x4_t hv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) hv[j] = g1[j * kSliceThreads + tid];
#pragma unroll
    for (int j = 0; j < NV; ++j) ((u32x4_t*)h1)[j * kSliceThreads + tid] = hv[j];
  }
  __syncthreads();
  block_find_digit<kLeD1Bins>(h1, (uint32_t)a.budget, pick);
  const uint32_t d1 = pick[0], rem = (uint32_t)a.budget - pick[1];
  const bool whole = rem == pick[2];
  uint32_t gt = 0u, in = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = (valid >> e) & 1u;
    const uint32_t b = (x[e] >> kLeD1Shift) & (uint32_t)(kLeD1Bins - 1);
    gt += ok && (b > d1 || (whole && b == d1));
    in |= (uint32_t)(ok && !whole && b == d1) << e;
  }
  uint32_t tot;
  uint32_t pos = block_exclusive_scan<kSliceThreads>((gt << 16) | __popc(in), &tot, wsum) & 0xffffu;
  const size_t cbase = ((size_t)grp * a.nst + sg) * kSlice;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((in >> e) & 1u) {
      a.cval[cbase + pos] = x[e];
      a.cidx[cbase + pos] = i0 + e;
      ++pos;
    }
  }
  if (tid == 0) {
    a.gtc[(size_t)grp * a.nst + sg] = tot >> 16;
    a.candc[(size_t)grp * a.nst + sg] = tot & 0xffffu;
    if (sg == 0) {
      uint32_t* pr = a.params + (size_t)grp * 4;
      pr[0] = d1 << kLeD1Shift;
      pr[1] = rem;
      pr[2] = whole ? 1u : 0u;
      pr[3] = kLeD1Bits;
    }
  }
}

// Head groups (a selection over all KV heads of a sequence: a group holds
// hg times the candidates, too many in one 12-bit bin): the second digit is
// settled from global histograms before the compaction, so le_emit starts
// from a 22-bit prefix.  lg_hist2: every slice settles the first digit and
// adds the bits 18..9 of its scores in that bin to the group's second-digit
// histogram.  lg_cand: every slice settles both digits, counts its scores
// above the 22-bit prefix and compacts the ones sharing it with their keys
// h*S + position, in position order.
__device__ __forceinline__ uint32_t* le_hist2_of(const SelArgs& a, int grp) {
  return a.hist1 + (size_t)gridDim.y * kLeD1Bins + (size_t)grp * kLeD2Bins;
}

__global__ void __launch_bounds__(kSliceThreads) lg_hist2(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kLeD1Bins];
  __shared__ uint32_t hist[kLeD2Bins];
  __shared__ uint32_t pick[3];
  const int grp = blockIdx.y, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, blockIdx.x);
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  {
    constexpr int NV = kLeD1Bins / (4 * kSliceThreads);
    const u32x4_t* g1 = (const u32x4_t*)(a.hist1 + (size_t)grp * kLeD1Bins);
    u32x4_t hv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) hv[j] = g1[j * kSliceThreads + tid];
#pragma unroll
    for (int j = 0; j < NV; ++j) ((u32x4_t*)h1)[j * kSliceThreads + tid] = hv[j];
  }
  for (int i = tid; i < kLeD2Bins; i += kSliceThreads) hist[i] = 0u;
  __syncthreads();
  block_find_digit<kLeD1Bins>(h1, (uint32_t)a.budget, pick);
  const uint32_t d1 = pick[0];
  if ((uint32_t)a.budget - pick[1] == pick[2]) return;   // d1's bin kept whole
  uint32_t bin[kPerThread];
  uint32_t act = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    bin[e] = (x[e] >> kLeD2Shift) & (uint32_t)(kLeD2Bins - 1);
    act |= (uint32_t)(((valid >> e) & 1u) &&
                      ((x[e] >> kLeD1Shift) & (uint32_t)(kLeD1Bins - 1)) == d1) << e;
  }
  hist_add_runs(hist, bin, act);
  __syncthreads();
  uint32_t* g2 = le_hist2_of(a, grp);
  for (int i = tid; i < kLeD2Bins; i += kSliceThreads)
    if (hist[i]) atomicAdd(&g2[i], hist[i]);
}

__global__ void __launch_bounds__(kSliceThreads) lg_cand(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kLeD1Bins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[kLeD2Bins];
  __shared__ uint32_t wsum[kSliceThreads / 64];
  __shared__ uint32_t pick[3];
  const int grp = blockIdx.y, sg = blockIdx.x, tid = threadIdx.x;
  const SliceAt at = slice_at(a, grp, sg);
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * kPerThread;
  uint32_t x[kPerThread];
  const uint32_t valid = load16(u, i0, a.lo, a.hi, x);
  {
    constexpr int NV = kLeD1Bins / (4 * kSliceThreads);
    const u32x4_t* g1 = (const u32x4_t*)(a.hist1 + (size_t)grp * kLeD1Bins);
    const u32x4_t* g2 = (const u32x4_t*)le_hist2_of(a, grp);
    u32x4_t hv[NV], hw;
#pragma unroll
    for (int j = 0; j < NV; ++j) hv[j] = g1[j * kSliceThreads + tid];
    hw = g2[tid];   // kLeD2Bins = 4 * kSliceThreads
#pragma unroll
    for (int j = 0; j < NV; ++j) ((u32x4_t*)h1)[j * kSliceThreads + tid] = hv[j];
    ((u32x4_t*)h2)[tid] = hw;
  }
  __syncthreads();
  block_find_digit<kLeD1Bins>(h1, (uint32_t)a.budget, pick);
  uint32_t rem = (uint32_t)a.budget - pick[1];
  uint32_t prefix = pick[0] << kLeD1Shift;
  uint32_t pmask = (uint32_t)(kLeD1Bins - 1) << kLeD1Shift;
  bool whole = rem == pick[2];
  int bits = kLeD1Bits;
  __syncthreads();
  if (!whole) {
    block_find_digit<kLeD2Bins>(h2, rem, pick);
    rem -= pick[1];
    prefix |= pick[0] << kLeD2Shift;
    pmask |= (uint32_t)(kLeD2Bins - 1) << kLeD2Shift;
    whole = rem == pick[2];
    bits = kLeD1Bits + kLeD2Bits;
    __syncthreads();
  }
  const uint32_t key0 = (uint32_t)(at.h * a.S + i0);
  uint32_t gt = 0u, in = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = (valid >> e) & 1u;
    const uint32_t m = x[e] & pmask;
    gt += ok && (m > prefix || (whole && m == prefix));
    in |= (uint32_t)(ok && !whole && m == prefix) << e;
  }
  uint32_t tot;
  uint32_t pos = block_exclusive_scan<kSliceThreads>((gt << 16) | __popc(in), &tot, wsum) & 0xffffu;
  const size_t cbase = ((size_t)grp * a.nst + sg) * kSlice;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((in >> e) & 1u) {
      a.cval[cbase + pos] = x[e];
      a.cidx[cbase + pos] = (int32_t)(key0 + e);
      ++pos;
    }
  }
  if (tid == 0) {
    a.gtc[(size_t)grp * a.nst + sg] = tot >> 16;
    a.candc[(size_t)grp * a.nst + sg] = tot & 0xffffu;
    if (sg == 0) {
      uint32_t* pr = a.params + (size_t)grp * 4;
      pr[0] = prefix;
      pr[1] = rem;
      pr[2] = whole ? 1u : 0u;
      pr[3] = (uint32_t)bits;
    }
  }
}

// le_emit runs 1024 threads per slice: thread t takes candidates
// [c*kLeR, (c+1)*kLeR) of slice t / TPS (c = t mod TPS, TPS threads per
// slice, a power of two), so the row's candidates come straight from their
// slices' regions into registers, with the counts and this slice's scores in
// the same round trip.  Thread order is slice order, and slice order with
// chunk order is position order, so one scan over threads orders the ties.
// A row with more candidates in one slice than its threads hold takes the
// general path: the candidates gathered into LDS (or read from global
// memory on every pass when there are too many), numbered in position order.
constexpr int kLeEmitThreads = 1024;
constexpr int kLeR = 8;

__global__ void __launch_bounds__(kLeEmitThreads) le_emit(SelArgs a, int tps_log2) {
  constexpr int NT = kLeEmitThreads, PT = kSlice / NT;
  static_assert(PT == 4, "four scores of the slice per thread");
  __shared__ uint32_t lval[kLeCandCap];
  __shared__ int32_t lidx[kLeCandCap];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kLeD2Bins];
  __shared__ uint32_t cstart[kLeMaxSlices];
  __shared__ uint32_t kept[kLeMaxSlices];
  __shared__ uint32_t wsum[2 * NT / 64];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t tval[64];
  __shared__ int32_t tkey[64];
  __shared__ uint32_t cut_s, val_s, over_s, tcnt;
  __shared__ uint32_t pb[kMaxWgHeads + 1];
  const int grp = blockIdx.y, sg = blockIdx.x, tid = threadIdx.x;
  const int ns = a.nst;
  const int tps = 1 << tps_log2;
  const int s_t = tid >> tps_log2, c_t = tid & (tps - 1);
  const bool has_slice = s_t < ns;
  // One round trip: the row's digit, this thread's slice counts and
  // candidates, this slice's four scores of this thread.
  const uint32_t* pr = a.params + (size_t)grp * 4;
  uint32_t prefix = pr[0];
  uint32_t rem = pr[1];
  const bool whole1 = pr[2] != 0u;       // the settled prefix's bin is kept whole
  const bool two = pr[3] != (uint32_t)kLeD1Bits;   // 22 bits settled (head groups)
  uint32_t pmask = two ? ((1u << (kLeD1Bits + kLeD2Bits)) - 1u) << kLeD2Shift
                       : (uint32_t)(kLeD1Bins - 1) << kLeD1Shift;
  const size_t srow = (size_t)grp * ns;
  const uint32_t cnt_t = has_slice ? a.candc[srow + s_t] : 0u;
  const uint32_t gt_t = (has_slice && c_t == 0) ? a.gtc[srow + s_t] : 0u;
  uint32_t cv[kLeR];
  int32_t ci[kLeR];
  {
    const int j0 = min(c_t * kLeR, kSlice - kLeR);
    const size_t rb = (srow + (has_slice ? s_t : 0)) * kSlice + j0;
    const u32x4_t* pv = (const u32x4_t*)(a.cval + rb);
    const u32x4_t* pi = (const u32x4_t*)(a.cidx + rb);
#pragma unroll
    for (int h = 0; h < kLeR / 4; ++h) {
      const u32x4_t w = pv[h], z = pi[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cv[4 * h + e] = w[e];
        ci[4 * h + e] = (int32_t)z[e];
      }
    }
  }
  const SliceAt at = slice_at(a, grp, sg);
  const uint32_t* u = (const uint32_t*)a.pooled + (size_t)at.row * a.S;
  const int i0 = slice_base(a, at.row) + at.sl * kSlice + tid * PT;
  const uint32_t key0 = (uint32_t)(at.h * a.S + i0);
  uint32_t x[PT];
  uint32_t valid = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const int i = i0 + e;
    valid |= (uint32_t)(i >= a.lo && i < a.hi) << e;
  }
  if (valid == 0xfu) {
    const u32x4_t w = *(const u32x4_t*)(u + i0);
#pragma unroll
    for (int e = 0; e < PT; ++e) x[e] = w[e];
  } else {
#pragma unroll
    for (int e = 0; e < PT; ++e) x[e] = ((valid >> e) & 1u) ? u[i0 + e] : 0u;
  }
  // Candidates this thread holds (its chunk of its slice), and whether any
  // slice has more than its threads hold.
  const uint32_t j0 = (uint32_t)c_t * kLeR;
  const uint32_t nmine = cnt_t > j0 ? min(cnt_t - j0, (uint32_t)kLeR) : 0u;
  if (tid == 0) {
    cut_s = 0xffffffffu;
    over_s = 0u;
    tcnt = 0u;
  }
  __syncthreads();
  if (has_slice && c_t == 0 && cnt_t > (uint32_t)tps * kLeR) over_s = 1u;
  __syncthreads();
  // This thread's share of the picks of the slices before this one (the
  // output offset of this slice is their sum).
  uint32_t off_part = 0u;
  if (!whole1 && !over_s) {
    // Register path.  Second digit (bits 18..9) unless already settled:
    // runs of equal bins among a thread's consecutive candidates cost one
    // atomic.
    uint32_t act = (1u << nmine) - 1u;
    uint32_t bin[kLeR];
    uint32_t nshare;
    bool whole;
    if (!two) {
      for (int i = tid; i < kLeD2Bins; i += NT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kLeR; ++r) bin[r] = (cv[r] >> kLeD2Shift) & (uint32_t)(kLeD2Bins - 1);
      hist_add_runs(hist, bin, act);
      __syncthreads();
      block_find_digit<kLeD2Bins>(hist, rem, pick);
      rem -= pick[1];
      prefix |= pick[0] << kLeD2Shift;
      pmask |= (uint32_t)(kLeD2Bins - 1) << kLeD2Shift;
      nshare = pick[2];
      whole = rem == nshare;
      __syncthreads();
    } else {
      uint32_t tot;
      block_exclusive_scan<NT>(nmine, &tot, wsum);
      nshare = tot;
      whole = rem == nshare;
    }
    if (!whole && nshare <= 64u) {
      // Few candidates share the 22-bit prefix (typically one max-pooled
      // plateau): rank them directly by (score desc, position asc); the
      // rem-th gives the exact score and the tie cut.
#pragma unroll
      for (int r = 0; r < kLeR; ++r) {
        if (((act >> r) & 1u) && (cv[r] & pmask) == prefix) {
          const uint32_t slot = atomicAdd(&tcnt, 1u);
          tval[slot] = cv[r] & kLeFullMask;
          tkey[slot] = ci[r];
        }
      }
      __syncthreads();
      if (tid < 64) {
        const uint32_t v = tid < (int)nshare ? tval[tid] : 0u;
        const int32_t kk = tid < (int)nshare ? tkey[tid] : 0;
        uint32_t rank = 0u;
#pragma unroll 8
        for (uint32_t j = 0; j < nshare; ++j) {
          const uint32_t vj = tval[j];
          rank += vj > v || (vj == v && tkey[j] < kk);
        }
        if (tid < (int)nshare && rank == rem - 1u) {
          val_s = v;
          cut_s = (uint32_t)kk;
        }
      }
      __syncthreads();
      prefix = val_s;
      pmask = kLeFullMask;
    } else if (!whole) {
      // Last digit (bits 8..0) over the candidates sharing the 22-bit prefix.
      for (int i = tid; i < kLeD3Bins; i += NT) hist[i] = 0u;
      __syncthreads();
      uint32_t act3 = 0u;
#pragma unroll
      for (int r = 0; r < kLeR; ++r) {
        bin[r] = cv[r] & (uint32_t)(kLeD3Bins - 1);
        act3 |= (uint32_t)(((act >> r) & 1u) && (cv[r] & pmask) == prefix) << r;
      }
      hist_add_runs(hist, bin, act3);
      __syncthreads();
      block_find_digit<kLeD3Bins>(hist, rem, pick);
      rem -= pick[1];
      prefix |= pick[0];
      pmask = kLeFullMask;
      whole = rem == pick[2];
      __syncthreads();
      if (!whole) {
        // Tie cut: the position of the rem-th candidate equal to the prefix,
        // counting in thread order (= position order).
        uint32_t neq = 0u;
#pragma unroll
        for (int r = 0; r < kLeR; ++r)
          neq += ((act >> r) & 1u) && (cv[r] & kLeFullMask) == prefix;
        uint32_t tot;
        uint32_t seen = block_exclusive_scan<NT>(neq, &tot, wsum);
        if (seen < rem && rem <= seen + neq) {
#pragma unroll
          for (int r = 0; r < kLeR; ++r) {
            if (((act >> r) & 1u) && (cv[r] & kLeFullMask) == prefix && ++seen == rem)
              cut_s = (uint32_t)ci[r];
          }
        }
        __syncthreads();
      }
    }
    const uint32_t cut = cut_s;
    if (s_t < sg) {
      uint32_t nk = gt_t;
#pragma unroll
      for (int r = 0; r < kLeR; ++r) {
        const uint32_t m = cv[r] & pmask;
        nk += ((act >> r) & 1u) && (m > prefix || (m == prefix && (uint32_t)ci[r] <= cut));
      }
      off_part = nk;
    }
  } else if (whole1) {
    off_part = s_t < sg ? gt_t : 0u;
  } else {
    // General path: flat numbering of the candidates in position order.
    static_assert(kLeMaxSlices <= NT, "one slice count per thread");
    const uint32_t c1 = tid < ns ? a.candc[srow + tid] : 0u;
    kept[tid] = tid < ns ? a.gtc[srow + tid] : 0u;
    uint32_t ncand;
    const uint32_t ex = block_exclusive_scan<NT>(c1, &ncand, wsum);
    if (tid < ns) cstart[tid] = ex;
    __syncthreads();
    const uint32_t* cvg = a.cval + srow * kSlice;
    const int32_t* cig = a.cidx + srow * kSlice;
    const bool in_lds = ncand <= (uint32_t)kLeCandCap;
    if (in_lds) {
      for (uint32_t k = tid; k < ncand; k += NT) {
        const int sl = slice_of(cstart, ns, k);
        const size_t o = (size_t)sl * kSlice + (k - cstart[sl]);
        lval[k] = cvg[o];
        lidx[k] = cig[o];
      }
    }
    for (int i = tid; i < kLeD2Bins; i += NT) hist[i] = 0u;
    __syncthreads();
    auto cand = [&](uint32_t k, uint32_t& v, int32_t& i) {
      if (in_lds) {
        v = lval[k];
        i = lidx[k];
      } else {
        const int sl = slice_of(cstart, ns, k);
        const size_t o = (size_t)sl * kSlice + (k - cstart[sl]);
        v = cvg[o];
        i = cig[o];
      }
    };
    bool whole = false;
    if (!two) {
      for (uint32_t k0 = 0; k0 < ncand; k0 += NT) {
        const uint32_t k = k0 + tid;
        uint32_t v = 0u;
        int32_t key;
        if (k < ncand) cand(k, v, key);
        hist_add(hist, (v >> kLeD2Shift) & (uint32_t)(kLeD2Bins - 1), k < ncand);
      }
      __syncthreads();
      block_find_digit<kLeD2Bins>(hist, rem, pick);
      rem -= pick[1];
      prefix |= pick[0] << kLeD2Shift;
      pmask |= (uint32_t)(kLeD2Bins - 1) << kLeD2Shift;
      whole = rem == pick[2];
      __syncthreads();
    }
    if (!whole) {
      for (int i = tid; i < kLeD3Bins; i += NT) hist[i] = 0u;
      __syncthreads();
      for (uint32_t k0 = 0; k0 < ncand; k0 += NT) {
        const uint32_t k = k0 + tid;
        uint32_t v = 0u;
        int32_t key;
        if (k < ncand) cand(k, v, key);
        hist_add(hist, v & (uint32_t)(kLeD3Bins - 1), k < ncand && (v & pmask) == prefix);
      }
      __syncthreads();
      block_find_digit<kLeD3Bins>(hist, rem, pick);
      rem -= pick[1];
      prefix |= pick[0];
      pmask = kLeFullMask;
      whole = rem == pick[2];
      __syncthreads();
      if (!whole) {
        const uint32_t per = (ncand + NT - 1) / NT;
        const uint32_t k0 = tid * per, k1 = min(ncand, k0 + per);
        uint32_t neq = 0u;
        for (uint32_t k = k0; k < k1; ++k) {
          uint32_t v;
          int32_t key;
          cand(k, v, key);
          neq += (v & kLeFullMask) == prefix;
        }
        uint32_t tot;
        uint32_t seen = block_exclusive_scan<NT>(neq, &tot, wsum);
        if (seen < rem && rem <= seen + neq) {
          for (uint32_t k = k0; k < k1; ++k) {
            uint32_t v;
            int32_t key;
            cand(k, v, key);
            if ((v & kLeFullMask) == prefix && ++seen == rem) {
              cut_s = (uint32_t)key;
              break;
            }
          }
        }
        __syncthreads();
      }
    }
    const uint32_t cut = cut_s;
    for (uint32_t k0 = 0; k0 < ncand; k0 += NT) {
      const uint32_t k = k0 + tid;
      bool keep = false;
      int sl = 0;
      if (k < ncand) {
        uint32_t v;
        int32_t key;
        cand(k, v, key);
        const uint32_t m = v & pmask;
        keep = m > prefix || (m == prefix && (uint32_t)key <= cut);
        const int kh = key / a.S, kp = key - kh * a.S;
        sl = kh * a.ns + (kp - slice_base(a, grp * a.hg + kh)) / kSlice;
      }
      hist_add(kept, (uint32_t)sl, keep);
    }
    __syncthreads();
    off_part = tid < sg ? kept[tid] : 0u;
  }
  const uint32_t cut = cut_s;
  uint32_t keep = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const uint32_t m = x[e] & pmask;
    const bool k = ((valid >> e) & 1u) &&
                   (m > prefix || (m == prefix && key0 + e <= cut));
    keep |= (uint32_t)k << e;
  }
  uint32_t off, npick;
  const uint32_t pos0 = block_scan_pair<NT>(off_part, __popc(keep), &off, &npick, wsum);
  uint32_t pos = pos0 + off;
  int32_t* row = a.idx + (size_t)grp * a.n_keep;
  int32_t* out = row + at.h * (a.n_sink + a.W) + a.n_sink;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    if ((keep >> e) & 1u) {
      if (pos < (uint32_t)a.budget) out[pos] = i0 + e;
      ++pos;
    }
  }
  if (sg != 0) return;
  // Slice 0 of the group also writes every head's sinks and window and the
  // head offsets: head h's rows start at h*(n_sink+W) + (picks of the heads
  // before it), which needs the picks of every slice.
  if (!whole1 && !over_s) {
    kept[tid] = 0u;
    __syncthreads();
    if (has_slice) {
      uint32_t nk = gt_t;
#pragma unroll
      for (int r = 0; r < kLeR; ++r) {
        const uint32_t m = cv[r] & pmask;
        nk += (r < (int)nmine) && (m > prefix || (m == prefix && (uint32_t)ci[r] <= cut));
      }
      if (nk) atomicAdd(&kept[s_t], nk);
    }
    __syncthreads();
  } else if (whole1) {
    kept[tid] = tid < ns ? a.gtc[srow + tid] : 0u;
    __syncthreads();
  }
  {
    const uint32_t kt = tid < ns ? kept[tid] : 0u;
    uint32_t tot;
    const uint32_t exs = block_exclusive_scan<NT>(kt, &tot, wsum);
    const int h = tid / a.ns;
    if (tid < ns && tid == h * a.ns) pb[h] = min(exs, (uint32_t)a.budget);
    if (tid == 0) pb[a.hg] = (uint32_t)a.budget;
    __syncthreads();
  }
  const int seg = a.n_sink + a.W;
  if (a.head_off)
    for (int h = tid; h <= a.hg; h += NT)
      a.head_off[(size_t)grp * (a.hg + 1) + h] = (int32_t)(h * seg + pb[h]);
  for (int t = tid; t < a.hg * seg; t += NT) {
    const int h = t / seg, j = t - h * seg;
    const uint32_t start = h * seg + pb[h];
    if (j < a.n_sink) row[start + j] = j;
    else row[start + a.n_sink + (pb[h + 1] - pb[h]) + (j - a.n_sink)] = a.S - a.W + (j - a.n_sink);
  }
}

// Threads per slice in le_emit: the largest power of two with every slice
// of a row covered by the workgroup and a slice's region not overrun.
int le_tps_log2(int nst) {
  int t = 0;
  while ((2 << t) * nst <= kLeEmitThreads && (2 << t) * kLeR <= kSlice) ++t;
  return t;
}

// Arguments of the sliced kernels for one launch sequence.
SelArgs sel_args(const kvsel_desc& d, const SelectPlan& p, const float* pooled, int budget,
                 int32_t* idx, int32_t* head_off, char* ws) {
  const int seg = d.n_sink + d.obs_window;
  SelArgs a;
  a.pooled = pooled;
  a.idx = idx;
  a.head_off = head_off;
  a.hist1 = (uint32_t*)(ws + p.off_hist);
  a.hist2 = a.hist1 + (size_t)p.groups * kD1Bins;
  a.gtc = (uint32_t*)(ws + p.off_gtc);
  a.candc = (uint32_t*)(ws + p.off_candc);
  a.offs = (uint32_t*)(ws + p.off_offs);
  a.params = (uint32_t*)(ws + p.off_params);
  a.cval = (uint32_t*)(ws + p.off_cval);
  a.cidx = (int32_t*)(ws + p.off_cidx);
  a.S = d.seq_len;
  a.lo = d.n_sink;
  a.hi = d.seq_len - d.obs_window;
  a.budget = budget;
  a.n_sink = d.n_sink;
  a.W = d.obs_window;
  a.ns = p.ns;
  a.hg = p.hg;
  a.nst = p.ns * p.hg;
  a.n_keep = p.hg * seg + budget;
  return a;
}

}  // namespace

bool plan_select(const kvsel_desc& d, int budget, int hg, SelectPlan* p) {
  const int groups = d.batch * d.n_kv_heads / hg;
  const int lo = d.n_sink, hi = d.seq_len - d.obs_window;
  const long ncand = (long)hi - lo;
  // Single workgroup per group when the group's slices of 16 scores fit two
  // register batches of 512 threads (16K scores); otherwise the sliced
  // multi-workgroup kernels (the slice count includes the alignment lead-in;
  // sel_resolve keeps per-slice counters for at most kMaxGroupSlices slices
  // of a group).  One workgroup over 64K scores measured slower than the
  // sliced kernels (58 vs 33 us for eight 64K rows): its histogram atomics
  // and passes all run on one CU.
  const long nsl = (ncand + 3 + kPerThread - 1) / kPerThread;
  const bool single = nsl * hg <= 2L * 512;
  const long ns = (ncand + 3 + kSlice - 1) / kSlice;
  p->hg = hg;
  p->groups = groups;
  p->nsl = (int)nsl;
  if (hg > kMaxWgHeads) return false;
  if (hg == 1) {
    p->multi = budget > 0 && !single && ns <= kMaxGroupSlices;
  } else {
    if (!single && ns * hg > kMaxGroupSlices) return false;
    p->multi = budget > 0 && !single;
  }
  p->ns = p->multi ? (int)ns : 0;
  const size_t nst = (size_t)p->ns * hg;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  if (p->multi) {
    // both digit histograms of the generic select, or the layer-end
    // chain's 12-bit first-digit histogram
    p->off_hist = take((size_t)groups * max(kD1Bins + kD2Bins, kLeD1Bins + kLeD2Bins) * 4);
    p->off_gtc = take((size_t)groups * nst * 4);
    p->off_candc = take((size_t)groups * nst * 4);
    p->off_offs = take((size_t)groups * nst * 4);
    p->off_params = take((size_t)groups * 4 * 4);
    p->off_cval = take((size_t)groups * nst * kSlice * 4);
    p->off_cidx = take((size_t)groups * nst * kSlice * 4);
  }
  p->total = off;
  return true;
}

kvsel_status launch_select(const kvsel_desc& d, const SelectPlan& p, const float* pooled,
                           int budget, int32_t* idx, int32_t* head_off, char* ws,
                           hipStream_t stream) {
  const int hg = p.hg, groups = p.groups;
  const int seg = d.n_sink + d.obs_window;
  const int n_keep = hg * seg + budget;
  const int lo = d.n_sink, hi = d.seq_len - d.obs_window;
  if (!p.multi) {
    // Smallest block whose register batches hold the group (16 scores per
    // thread): no idle threads on short rows, fewer waves at each barrier.
    const long tot = (long)p.nsl * hg;
    const dim3 g(groups);
    const GatherArgs none = {nullptr, nullptr, nullptr, nullptr, 0, 1};
#define KVSEL_SELECT_1WG(NT, NB)                                                              \
  KVSEL_LAUNCH("select_kernel", (select_kernel<NT, NB, false>), g, dim3(NT), 0, stream, pooled, idx,      \
                     head_off, d.seq_len, lo, hi, budget, d.n_sink, d.obs_window, n_keep, hg, \
                     p.nsl, none)
    if (tot <= 256) KVSEL_SELECT_1WG(256, 1);
    else if (tot <= 512) KVSEL_SELECT_1WG(512, 1);
    else KVSEL_SELECT_1WG(512, 2);   // beyond 1024 slices: later batches reloaded
#undef KVSEL_SELECT_1WG
    return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
  }
  SelArgs a = sel_args(d, p, pooled, budget, idx, head_off, ws);
  const dim3 sg(a.nst, groups);
  if (a.nst <= kLeMaxSlices) {
    // the select of the layer-end path: one KV-head row per group settles a
    // 12-bit digit before the compaction, a head group 22 bits (its group
    // holds hg rows of candidates)
    KVSEL_LAUNCH("le_init", le_init, dim3(groups), dim3(256), 0, stream, a);
    KVSEL_LAUNCH("le_hist", le_hist, sg, dim3(kSliceThreads), 0, stream, a);
    if (hg == 1) {
      KVSEL_LAUNCH("le_cand", le_cand, sg, dim3(kSliceThreads), 0, stream, a);
    } else {
      KVSEL_LAUNCH("lg_hist2", lg_hist2, sg, dim3(kSliceThreads), 0, stream, a);
      KVSEL_LAUNCH("lg_cand", lg_cand, sg, dim3(kSliceThreads), 0, stream, a);
    }
    KVSEL_LAUNCH("le_emit", le_emit, sg, dim3(kLeEmitThreads), 0, stream, a, le_tps_log2(a.nst));
    return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
  }
  KVSEL_LAUNCH("sel_init", sel_init, dim3(groups), dim3(256), 0, stream, a);
  KVSEL_LAUNCH("sel_hist", sel_hist, sg, dim3(kSliceThreads), 0, stream, a);
  KVSEL_LAUNCH("sel_hist2", sel_hist2, sg, dim3(kSliceThreads), 0, stream, a);
  KVSEL_LAUNCH("sel_cand", sel_cand, sg, dim3(kSliceThreads), 0, stream, a);
  KVSEL_LAUNCH("sel_resolve", sel_resolve, dim3(groups), dim3(kSelThreads), 0, stream, a);
  KVSEL_LAUNCH("sel_emit", sel_emit, sg, dim3(kSliceThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}


kvsel_status launch_select_compact(const kvsel_desc& d, const SelectPlan& p, const float* pooled,
                                   int budget, int32_t* idx, const void* k, const void* v,
                                   void* k_out, void* v_out, char* ws, hipStream_t stream) {
  const int seg = d.n_sink + d.obs_window;
  const int n_keep = seg + budget;
  const int e = d.dtype == KVSEL_F32 ? 4 : 2;
  if (p.multi || p.hg != 1 || n_keep > kMaxFusedKeep) {
    const kvsel_status st = launch_select(d, p, pooled, budget, idx, nullptr, ws, stream);
    if (st != KVSEL_OK) return st;
    return launch_compact(d, k, v, idx, n_keep, k_out, v_out, stream);
  }
  // Enough replicas to spread the gather over the chip, at least 16 rows each.
  int reps = 256 / p.groups;
  if (reps > n_keep / 16) reps = n_keep / 16;
  if (reps < 1) reps = 1;
  GatherArgs ga;
  ga.k = (const u32x4_t*)k;
  ga.v = (const u32x4_t*)v;
  ga.ko = (u32x4_t*)k_out;
  ga.vo = (u32x4_t*)v_out;
  ga.vpr = d.head_dim * e / 16;
  ga.reps = reps;
  const int lo = d.n_sink, hi = d.seq_len - d.obs_window;
  const long tot = (long)p.nsl;
  const dim3 g(p.groups * reps);
#define KVSEL_SELECT_GATHER(NT, NB)                                                          \
  KVSEL_LAUNCH("select_kernel", (select_kernel<NT, NB, true>), g, dim3(NT), 0, stream, pooled, idx,      \
                     (int32_t*)nullptr, d.seq_len, lo, hi, budget, d.n_sink, d.obs_window,    \
                     n_keep, 1, p.nsl, ga)
  if (tot <= 256) KVSEL_SELECT_GATHER(256, 1);
  else if (tot <= 512) KVSEL_SELECT_GATHER(512, 1);
  else KVSEL_SELECT_GATHER(512, 2);
#undef KVSEL_SELECT_GATHER
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

// The first-digit histograms of every group, then (head groups) the
// second-digit ones: one contiguous run of words to clear.
uint32_t* select_hists(const SelectPlan& p, char* ws, size_t* words) {
  *words = (size_t)p.groups * (p.hg > 1 ? kLeD1Bins + kLeD2Bins : kLeD1Bins);
  return (uint32_t*)(ws + p.off_hist);
}

bool layer_end_fusable(const kvsel_desc& d, const SelectPlan& p, int budget, int pool_kernel) {
  const long ncand = (long)d.seq_len - d.obs_window - d.n_sink;
  return p.multi && budget > 0 && (pool_kernel - 1) / 2 <= kMaxPoolHalo &&
         (long)p.ns * p.hg <= kLeMaxSlices && (long)budget <= (long)p.hg * ncand;
}

// The gather runs as its own evenly spread kernel after the emit: copying
// each slice's picks inside the emit left the slices that hold many picks
// (clustered scores) far behind the rest (15.8 us for emit + copy at 128K
// against 4.6 + 7.0 us for the two kernels).
kvsel_status launch_layer_end_select(const kvsel_desc& d, const SelectPlan& p, const float* raw,
                                     float* pooled, int pool_kernel, int budget, int32_t* idx,
                                     int32_t* head_off, const void* k, const void* v,
                                     void* k_out, void* v_out, char* ws, hipStream_t stream) {
  SelArgs a = sel_args(d, p, pooled, budget, idx, head_off, ws);
  const dim3 sg(a.nst, p.groups);
  KVSEL_LAUNCH("sel_pool_hist", sel_pool_hist, sg, dim3(kPoolThreads), 0, stream, a, raw, pooled,
               (pool_kernel - 1) / 2);
  if (p.hg == 1) {
    KVSEL_LAUNCH("le_cand", le_cand, sg, dim3(kSliceThreads), 0, stream, a);
  } else {
    KVSEL_LAUNCH("lg_hist2", lg_hist2, sg, dim3(kSliceThreads), 0, stream, a);
    KVSEL_LAUNCH("lg_cand", lg_cand, sg, dim3(kSliceThreads), 0, stream, a);
  }
  KVSEL_LAUNCH("le_emit", le_emit, sg, dim3(kLeEmitThreads), 0, stream, a, le_tps_log2(a.nst));
  if (hipGetLastError() != hipSuccess) return KVSEL_ERR_DEVICE;
  if (p.hg == 1) return launch_compact(d, k, v, idx, a.n_keep, k_out, v_out, stream);
  return launch_compact_flat(d, k, v, idx, head_off, a.n_keep, k_out, v_out, stream);
}

// Final index rows of the streaming path: sinks, then the positions of the
// selected list entries (selected in ascending list order, which is
// ascending position order), then the observation window.
__global__ void __launch_bounds__(256) stream_finish_kernel(const int32_t* __restrict__ sel,
                                                            const int32_t* __restrict__ cpos,
                                                            int32_t* __restrict__ idx, int M,
                                                            int budget, int n_sink, int W, int S) {
  const int row = blockIdx.y;
  const int n_keep = n_sink + budget + W;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n_keep) return;
  int32_t pos;
  if (r < n_sink) {
    pos = r;
  } else if (r < n_sink + budget) {
    const int32_t li = sel[(size_t)row * budget + (r - n_sink)];
    pos = (li >= 0 && li < M) ? cpos[(size_t)row * M + li] : -1;
  } else {
    pos = S - W + (r - n_sink - budget);
  }
  idx[(size_t)row * n_keep + r] = pos;
}

kvsel_status launch_stream_finish(const int32_t* sel, const int32_t* cpos, int32_t* idx,
                                  int rows, int M, int budget, int n_sink, int W, int S,
                                  hipStream_t stream) {
  const int n_keep = n_sink + budget + W;
  if (n_keep == 0) return KVSEL_OK;
  KVSEL_LAUNCH("stream_finish_kernel", stream_finish_kernel, dim3((n_keep + 255) / 256, rows),
               dim3(256), 0, stream, sel, cpos, idx, M, budget, n_sink, W, S);
  return hipGetLastError() == hipSuccess ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

}  // namespace kvsel
