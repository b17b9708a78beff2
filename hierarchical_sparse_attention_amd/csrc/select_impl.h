// select_impl.h - device code of stage 2 (block scoring, top-k, window),
// shared by the selection kernel and the fused select-and-decode kernel.
//
// Sources: "8x256K ... porting HiSparse to QSA" sections 2.2 (coarse level,
// fine level inside the kept coarse blocks, window level, merged), 3.2
// (selection moved to the GPU: block dot products then a top-k) and 5.1 (fp32
// scores compared at full precision); "SGLang hierarchical sparse attention"
// section 3.1.2 (Quest box bound); untitled HiSparse write-up section 3.3
// (window forced, then top-K in descending order).
//
// Work of one selection level is cut into workgroup tasks:
//  * scoring - HBM stream of the summary table. Per unit the G query heads
//    are folded into per-dimension coefficients once (sum of q for mean rows;
//    sum of the negative / positive parts of q for the min / max rows of a
//    box, since max(q m, q M) = m min(q,0) + M max(q,0)), so each summary
//    element costs one FMA whatever G is. A row is read by LPR lanes with
//    16-byte loads and reduced across them with DPP; fp32 scores go to the
//    workspace with device-coherent stores.
//  * top-k - one workgroup reads the unit's published scores and selects,
//    exactly, on order-preserving uint32 keys of the fp32 scores. With the
//    keys in registers (every path up to 4096 block candidates or 8192
//    token slots) an LDS histogram over the candidates' own value range
//    narrows the k-th largest key to a bucket, usually of a few keys, which
//    are then ranked directly (key descending, candidate index ascending:
//    the lowest-index tie-break); a crowded bucket is split again over its
//    own key range. Larger units take 11-bit radix passes over keys in LDS
//    or re-read from the scores. Kept blocks and the window's blocks are
//    written out as ascending ids (to LDS, to global memory, or both).
#pragma once

#include <type_traits>

#include "hs_internal.h"
#include "summ_impl.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int kUnroll = 16;  // summary rows in flight per lane group while scoring
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kBins / kThreads;
constexpr int kRegKeys = 16;    // keys per thread of the register path (<= 4096 candidates)
constexpr int kLdsKeys = 8192;  // beyond this many candidates keys stay in the workspace
constexpr int kMaxCand = 128;   // a threshold bin this small is ranked directly
static_assert(kMaxCand % 8 == 0, "bin ranking reads candidates in groups of 8");

// Number of scoring tasks of a unit for a level with n_slots_max candidates.
__host__ __device__ inline int select_chunks(int n_slots_max) {
  return (n_slots_max + kRowsPerWG - 1) / kRowsPerWG;
}

// slot c -> block id (or -1 if the slot holds no candidate)
struct SlotMap {
  const int32_t* gamma;
  int gcnt, ratio, nb;
  __device__ __forceinline__ int block_of(int c) const {
    if (gamma == nullptr) return c < nb ? c : -1;
    const int gi = c / ratio;
    if (gi >= gcnt) return -1;
    return from_entry(gamma[gi], c - gi * ratio);
  }
  // block of the slot at offset r of coarse entry g (-1 if none)
  __device__ __forceinline__ int from_entry(int g, int r) const {
    const int beta = g * ratio + r;
    return g >= 0 && beta < nb ? beta : -1;
  }
};

// Coarse entries of one scoring chunk staged in LDS, so that a row's block
// costs an LDS read instead of a dependent global load (a chunk of
// kRowsPerWG slots spans at most kRowsPerWG entries).
constexpr int kGammaLds = 512;

// What a unit looks like to one selection level: T (clamped), its number of
// blocks nb, its candidate slots and their count n.
struct UnitGeom {
  int T, nb, n;
  SlotMap slots;
};

// k of a unit: top_k, or max(1, int(nb * ratio)) with a ratio (nb * ratio is
// exact in double for a float ratio and nb < 2^24, so the floor is exact).
__device__ __forceinline__ int unit_top_k(const SelectParams& p, int nb) {
  if (p.top_k_ratio > 0.f) {
    const int k = (int)((double)nb * (double)p.top_k_ratio);
    return k > 1 ? k : 1;
  }
  return p.top_k;
}

__device__ __forceinline__ UnitGeom unit_geom(const SelectParams& p, int unit) {
  UnitGeom u;
  u.T = clamp_len(p.kv, unit / p.kv.num_kv_heads);
  const int nb = (u.T + p.block_size - 1) / p.block_size;
  u.nb = nb < p.out_blocks_max ? nb : p.out_blocks_max;
  u.slots.nb = u.nb;
  u.slots.ratio = p.ratio;
  u.slots.gamma = nullptr;
  u.slots.gcnt = 0;
  if (p.gamma) {
    int gc = p.gamma_cnt[unit];
    gc = gc < 0 ? 0 : (gc > p.gamma_cap ? p.gamma_cap : gc);
    u.slots.gamma = p.gamma + (int64_t)unit * p.gamma_cap;
    u.slots.gcnt = gc;
  }
  const int n = p.gamma ? u.slots.gcnt * p.ratio : u.nb;
  u.n = n < p.n_slots_max ? n : p.n_slots_max;
  return u;
}

template <typename TE>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (sizeof(TE) == 4) return reinterpret_cast<const float*>(base)[i];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

struct TopkShared {
  // bins, then one dummy bin per lane that absorbs the counts of absent keys
  __attribute__((aligned(16))) uint32_t hist[kBins + kWave];
  __attribute__((aligned(16))) float xpose[kThreads * kRegKeys];  // scores, transposed
  uint32_t cand_key[kWaves][kMaxCand];   // threshold-bin keys (up to kMaxCand + 7 read)
  int32_t cand_slot[kWaves][kMaxCand];
  int32_t cand_blk[kWaves][kMaxCand];    // their blocks (register path)
  uint32_t tie_cnt[kRegKeys][kWaves];
  __attribute__((aligned(16))) uint32_t scan_tot[3][kWaves];  // wave totals of three scans
  float stage[kRowsPerWG];                     // scores of this workgroup's rows
  __attribute__((aligned(16))) uint32_t wave_tot[kWaves];
  uint32_t red[3][kWaves];
  __attribute__((aligned(16))) uint32_t bcast[4];
  __attribute__((aligned(16))) uint32_t wcnt[kWaves];
  uint32_t kbits[kThreads * kRegKeys / 32];  // threshold-bin candidates ranked into the top-k
  uint32_t n_cand;                           // threshold-bin candidates gathered
  int last;
  int32_t gam[kGammaLds];                    // staged coarse entries (see kGammaLds)
};

// ----------------------------------------------------- wave-level scans (DPP)
// Row shifts and row broadcasts stay in the VALU (no LDS round trips):
// Hillis-Steele inside each 16-lane row with row_shr:1,2,4,8 (lanes without a
// source read the identity), then row_bcast:15 adds row 0's (row 2's) total to
// row 1 (row 3), and row_bcast:31 adds rows 0-1's total to rows 2 and 3.
template <int CTRL, int ROWS, uint32_t IDENTITY>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)IDENTITY, (int)x, CTRL, ROWS, 0xF, false);
}

struct OpAdd {
  static constexpr uint32_t id = 0u;
  __device__ static uint32_t f(uint32_t a, uint32_t b) { return a + b; }
};
struct OpMax {
  static constexpr uint32_t id = 0u;
  __device__ static uint32_t f(uint32_t a, uint32_t b) { return a > b ? a : b; }
};
struct OpMin {
  static constexpr uint32_t id = 0xFFFFFFFFu;
  __device__ static uint32_t f(uint32_t a, uint32_t b) { return a < b ? a : b; }
};

template <typename OP>
__device__ __forceinline__ uint32_t wave_incl_scan_op(uint32_t x) {
  x = OP::f(x, dpp_u<0x111, 0xF, OP::id>(x));  // row_shr:1
  x = OP::f(x, dpp_u<0x112, 0xF, OP::id>(x));  // row_shr:2
  x = OP::f(x, dpp_u<0x114, 0xF, OP::id>(x));  // row_shr:4
  x = OP::f(x, dpp_u<0x118, 0xF, OP::id>(x));  // row_shr:8
  x = OP::f(x, dpp_u<0x142, 0xA, OP::id>(x));  // row_bcast:15 -> rows 1, 3
  x = OP::f(x, dpp_u<0x143, 0xC, OP::id>(x));  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) { return wave_incl_scan_op<OpAdd>(x); }

// Reduction over the wave, the same value in every lane.
template <typename OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_op<OP>(x), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t x) { return wave_reduce<OpAdd>(x); }
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) { return wave_reduce<OpMax>(x); }
__device__ __forceinline__ uint32_t wave_min_u(uint32_t x) { return wave_reduce<OpMin>(x); }

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* total, TopkShared& sh) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == kWave - 1) sh.wave_tot[wave] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t v = sh.wave_tot[w];
    off += w < wave ? v : 0u;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return off + inc - x;
}

// Histogram bins are stored swizzled so that the digit search below reads
// them without LDS bank conflicts: logical bin b lives at (b % 8) * 256 + b / 8.
__device__ __forceinline__ int hist_slot(uint32_t b) { return (int)((b & 7u) * kThreads + (b >> 3)); }

// Digit search of one radix pass over the LDS histogram: thread t owns the
// logical bins nbins-1-8t down to nbins-8-8t; exactly one bin d has
// above(d) < remaining <= above(d) + hist[d]. Updates prefix and remaining in
// every thread and returns hist[d], the number of keys in the bin.
__device__ __forceinline__ uint32_t take_digit(TopkShared& sh, int nbins, int shift, uint32_t& prefix,
                                               uint32_t& remaining) {
  const int tid = thread_id();
  uint32_t h[kBinsPerThread], local = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    const int bin = nbins - 1 - (kBinsPerThread * tid + i);
    h[i] = bin >= 0 ? sh.hist[hist_slot((uint32_t)bin)] : 0u;
    local += h[i];
  }
  uint32_t tot;
  uint32_t above = block_excl_scan(local, &tot, sh);
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    if (h[i] && above < remaining && above + h[i] >= remaining) {
      sh.bcast[0] = (uint32_t)(nbins - 1 - (kBinsPerThread * tid + i));
      sh.bcast[1] = above;
      sh.bcast[2] = h[i];
    }
    above += h[i];
  }
  __syncthreads();
  prefix |= sh.bcast[0] << shift;
  remaining -= sh.bcast[1];
  const uint32_t in_bin = sh.bcast[2];
  __syncthreads();
  return in_bin;
}

__device__ __forceinline__ void mark(uint32_t* bitmap, int beta) {
  atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
}

// Exclusive prefix sum over the workgroup in thread order without a trailing
// barrier: tot4 (4 words of LDS, 16-byte aligned) holds the wave totals and
// must not be rewritten before every thread has passed a later barrier.
// *total gets the workgroup's sum.
__device__ __forceinline__ uint32_t wg_excl_scan(uint32_t x, uint32_t* tot4, uint32_t* total) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == kWave - 1) tot4[wave] = inc;
  __syncthreads();
  const uint4 t = *reinterpret_cast<const uint4*>(tot4);
  *total = t.x + t.y + t.z + t.w;
  return inc - x + (wave > 0 ? t.x : 0u) + (wave > 1 ? t.y : 0u) + (wave > 2 ? t.z : 0u);
}

// Digit search of a radix pass over the plain-layout LDS histogram: thread t
// owns the logical bins nbins-1-8t down to nbins-8-8t (two 16-byte loads); a
// workgroup scan of the threads' sums gives the count above each thread's
// bins, and the one thread holding the bin d with
// above(d) < remaining <= above(d) + hist[d] broadcasts it (the search
// itself is branch-free). Updates prefix and remaining in every thread and
// returns hist[d].
__device__ __forceinline__ uint32_t take_digit_flat(TopkShared& sh, int nbins, int shift,
                                                    uint32_t& prefix, uint32_t& remaining) {
  const int tid = thread_id();
  const int top = nbins - kBinsPerThread * tid;  // this thread's bins: [top - 8, top)
  uint32_t h[kBinsPerThread];
  if (nbins >= kBinsPerThread) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (top > 0) {
      a = *reinterpret_cast<const uint4*>(&sh.hist[top - 8]);
      b = *reinterpret_cast<const uint4*>(&sh.hist[top - 4]);
    }
    h[0] = b.w; h[1] = b.z; h[2] = b.y; h[3] = b.x;
    h[4] = a.w; h[5] = a.z; h[6] = a.y; h[7] = a.x;
  } else {
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) h[i] = top - 1 - i >= 0 ? sh.hist[top - 1 - i] : 0u;
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) local += h[i];
  uint32_t tot;
  uint32_t run = wg_excl_scan(local, sh.scan_tot[0], &tot);
  int hit = -1;
  uint32_t hit_above = 0, hit_h = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    const bool here = run < remaining && run + h[i] >= remaining;
    hit = here ? i : hit;
    hit_above = here ? run : hit_above;
    hit_h = here ? h[i] : hit_h;
    run += h[i];
  }
  if (hit >= 0) {
    sh.bcast[0] = (uint32_t)(top - 1 - hit);
    sh.bcast[1] = hit_above;
    sh.bcast[2] = hit_h;
  }
  __syncthreads();
  const uint4 bc = *reinterpret_cast<const uint4*>(sh.bcast);
  prefix |= bc.x << shift;
  remaining -= bc.y;
  return bc.z;
}

// The float whose order_key is k (+0 for the key of -0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Threshold of a workgroup's top k_eff keys (0 < k_eff < n_valid) by buckets
// over the candidates' own range. Thread t holds KPT keys kr (bit u of
// `present`: kr[u] is a candidate; kmin / kmax: the candidates' extreme
// keys). The first pass buckets linearly in value over [vmin, vmax] (rounded
// float arithmetic is monotone, and the keys spread over all the buckets, so
// the histogram's atomics rarely collide; a radix digit of the leading key
// bits would put them in a few exponent buckets). While the threshold's
// bucket holds more than kMaxCand candidates, the next pass buckets that
// bucket's own [min, max] in key order (fixed-width buckets from its min),
// which always splits it. Requires sh.hist[0, kBins) zero behind a barrier;
// uses sh.red[1..2], sh.scan_tot[0] and sh.bcast.
struct Threshold {
  uint32_t keep;       // candidates above the threshold's bucket (or the whole bucket, taken)
  uint32_t cand;       // the threshold bucket's candidates still to settle (modes 1, 2)
  uint32_t remaining;  // how many of them are kept
  uint32_t in_bin;     // their number over the workgroup
  int mode;            // 0: settled, 1: all equal (first `remaining` in slot order), 2: rank
};
template <int KPT>
__device__ __forceinline__ Threshold bucket_threshold(TopkShared& sh, const uint32_t (&kr)[KPT],
                                                      uint32_t present, uint32_t k_eff,
                                                      uint32_t n_valid, uint32_t kmin,
                                                      uint32_t kmax) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  Threshold th{0u, present, k_eff, n_valid, 0};
  uint32_t lo = kmin, hi = kmax;
  const float vlo = key_value(lo), width = key_value(hi) - vlo;
  const float vscale = (float)kBins / width;
  bool by_value = width > 0.f && __builtin_isfinite(width) && __builtin_isfinite(vscale);
  for (;;) {
    if (lo == hi) {
      th.mode = 1;
      return th;
    }
    // this pass's bucket of every candidate (the dummy bin of the lane for
    // the others); key buckets are (k - lo) >> sh_k with (hi - lo) >> sh_k
    // in [kBins / 2, kBins)
    const int sh_k = max(0, 32 - __clz(hi - lo) - kDigitBits);
    uint32_t bk[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const uint32_t b = by_value
          ? min((uint32_t)((key_value(kr[u]) - vlo) * vscale), (uint32_t)(kBins - 1))
          : (kr[u] - lo) >> sh_k;
      bk[u] = (th.cand >> u) & 1u ? b : (uint32_t)(kBins + lane);
      atomicAdd(&sh.hist[bk[u]], 1u);
    }
    __syncthreads();
    uint32_t d = 0;
    th.in_bin = take_digit_flat(sh, kBins, 0, d, th.remaining);
    uint32_t next = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {  // dummy bins are above every bucket but not candidates
      const bool c = (th.cand >> u) & 1u;
      th.keep |= (c && bk[u] > d ? 1u : 0u) << u;
      next |= (c && bk[u] == d ? 1u : 0u) << u;
    }
    th.cand = next;
    if (th.in_bin == th.remaining) {  // the whole bucket is kept
      th.keep |= th.cand;
      th.cand = 0;
      return th;
    }
    if (th.in_bin <= (uint32_t)kMaxCand) {
      th.mode = 2;
      return th;
    }
    // the bucket's own key range for the next pass
    uint32_t bmax = 0, bmin_inv = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool c = (th.cand >> u) & 1u;
      bmax = max(bmax, c ? kr[u] : 0u);
      bmin_inv = max(bmin_inv, c ? ~kr[u] : 0u);
    }
    bmax = wave_max_u(bmax);
    bmin_inv = wave_max_u(bmin_inv);
    if (lane == 0) {
      sh.red[1][wave] = bmax;
      sh.red[2][wave] = bmin_inv;
    }
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
    __syncthreads();
    hi = 0;
    lo = 0xFFFFFFFFu;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      hi = max(hi, sh.red[1][w2]);
      lo = min(lo, ~sh.red[2][w2]);
    }
    by_value = false;
  }
}

// Top-k, window and ascending ids of a single-level unit with at most
// kThreads * kRegKeys candidates (candidate c is block c), to `list` (LDS)
// and/or `gids` / `*gcnt` (global). Thread t owns the contiguous candidates
// c = kRegKeys * t + u (u < kRegKeys), keys in registers, so candidate order
// is thread order and every "rank in block order" below is one workgroup
// scan of a per-thread count. The key range comes with the scores (the
// scoring tasks publish each chunk's largest key and ~key), so the first
// radix pass starts right after the loads. Kept candidates (above the
// threshold, ranked into the top-k inside the threshold bin, or in the
// window) are bits of a per-thread mask. On this hardware a dependent LDS
// round trip costs about as much as 15 VALU instructions, so LDS reads are
// batched and per-key work is kept branch-free.
__device__ __forceinline__ int topk_single(const SelectParams& p, int unit, const UnitGeom& ug,
                                           TopkShared& sh, int32_t* list, int32_t* gids,
                                           int32_t* gcnt) {
  constexpr int KPT = kRegKeys;
  const int tid = thread_id();
  const int n = ug.n;
  const int c0 = KPT * tid;  // first candidate of this thread
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring
  float v[KPT];
  uint32_t kmax = 0, kmin_inv = 0;
  {
    // coalesced loads (thread t: candidates u * 256 + t), transposed through
    // LDS to the contiguous ownership; every chunk's key range in the same
    // round trip. Bounded by the capacity, not by n, so that they do not
    // wait for the load of the unit's length (chunks past n published empty
    // ranges; candidates past n are masked below).
    const int nmax = p.n_slots_max;
#pragma unroll
    for (int u = 0; u < KPT; ++u)  // unconditional (clamped) loads that overlap
      v[u] = published(&sc[min(u * kThreads + tid, nmax - 1)]);
    const int nch = select_chunks(nmax);
    const int32_t* ck = reinterpret_cast<const int32_t*>(p.chunk_keys + (int64_t)unit * nch * 2);
    for (int ch = tid; ch < nch; ch += kThreads) {
      kmax = max(kmax, (uint32_t)published_i32(&ck[2 * ch]));
      kmin_inv = max(kmin_inv, (uint32_t)published_i32(&ck[2 * ch + 1]));
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) sh.xpose[u * kThreads + tid] = v[u];
    kmax = wave_max_u(kmax);
    kmin_inv = wave_max_u(kmin_inv);
    if ((tid & (kWave - 1)) == 0) {
      sh.red[1][tid / kWave] = kmax;
      sh.red[2][tid / kWave] = kmin_inv;
    }
  }
  for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
  if (tid < kThreads * KPT / 32) sh.kbits[tid] = 0u;
  if (tid == 0) sh.n_cand = 0u;
  int w0 = ug.nb;  // blocks w0 .. nb-1 hold the window's tokens
  if (p.window > 0) {
    const int64_t lo_tok = (int64_t)ug.T - p.window;
    w0 = lo_tok <= 0 ? 0 : (int)(lo_tok / p.block_size);
  }
  __syncthreads();  // transposed scores, key ranges, cleared histogram and bits
  // caller-forced blocks: bits of the candidate bitmap, read back below
  const int32_t* forced = p.forced ? p.forced + (int64_t)unit * p.forced_cap : nullptr;
  for (int i = tid; i < p.forced_cap; i += kThreads) {
    const int f = forced[i];
    if (f >= 0 && f < n) atomicOr(&sh.kbits[f >> 5], 1u << (f & 31));
  }
  {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      kmax = max(kmax, sh.red[1][w]);
      kmin_inv = max(kmin_inv, sh.red[2][w]);
    }
#pragma unroll
    for (int u = 0; u < KPT; u += 4) {
      const float4 x = *reinterpret_cast<const float4*>(&sh.xpose[c0 + u]);
      v[u] = x.x;
      v[u + 1] = x.y;
      v[u + 2] = x.z;
      v[u + 3] = x.w;
    }
  }
  // keys; candidates past n get key 0 (below every finite score's key)
  uint32_t kr[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const uint32_t bits = __float_as_uint(v[u] + 0.f);  // -0 -> +0
    const uint32_t k = bits ^ ((uint32_t)((int32_t)bits >> 31) | 0x80000000u);
    kr[u] = c0 + u < n ? k : 0u;
  }
  const uint32_t kmin = ~kmin_inv;
  const uint32_t n_valid = n > 0 ? (uint32_t)n : 0u;
  const uint32_t k_eff = min((uint32_t)max(unit_top_k(p, ug.nb), 0), n_valid);
  // bit u of keep / cand: candidate c0 + u is kept / in the threshold's
  // bucket (present keys are never 0, so "present" is the candidate range)
  constexpr uint32_t kFull = (1u << KPT) - 1u;
  const auto from = [&](int lo) {  // bits u with c0 + u >= lo
    const int s = lo - c0;
    return s <= 0 ? kFull : (s >= KPT ? 0u : (kFull << s) & kFull);
  };
  const uint32_t present = kFull & ~from(n), in_window = from(w0);
  const bool keep_all = k_eff > 0 && k_eff == n_valid;
  Threshold th{0u, 0u, 0u, 0u, 0};
  if (k_eff > 0 && !keep_all)  // uniform
    th = bucket_threshold<KPT>(sh, kr, present, k_eff, n_valid, kmin, kmax);
  uint32_t keep = present & (keep_all ? kFull : (in_window | th.keep));
  if (p.forced_cap > 0) {  // uniform
    __syncthreads();  // every forced bit is set
    keep |= (sh.kbits[c0 >> 5] >> (c0 & 31)) & kFull & present;
  }
  const uint32_t inb = th.cand, remaining = th.remaining, in_bin = th.in_bin;
  if (th.mode == 1) {  // uniform
    // every key left equals the threshold: the first `remaining` of them in
    // candidate order are kept
    uint32_t m;
    uint32_t pos = wg_excl_scan((uint32_t)__popc(inb), sh.scan_tot[1], &m);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if ((inb >> u) & 1u) keep |= (pos++ < remaining ? 1u : 0u) << u;
  } else if (th.mode == 2) {  // uniform
    // at most kMaxCand keys: gather them (any order), rank each against all
    // of them (key desc, candidate asc) and set the bits of those ranked
    // below `remaining`
    uint32_t* ckey = &sh.cand_key[0][0];
    int32_t* cslot = &sh.cand_slot[0][0];
    for (uint32_t bits = inb; bits != 0; bits &= bits - 1) {  // usually no or one pass
      const int u = __builtin_ctz(bits);
      const uint32_t slot = atomicAdd(&sh.n_cand, 1u);
      const uint32_t vb = __float_as_uint(sh.xpose[c0 + u] + 0.f);  // the key of kr[u]
      ckey[slot] = vb ^ ((uint32_t)((int32_t)vb >> 31) | 0x80000000u);
      cslot[slot] = c0 + u;
    }
    __syncthreads();
    if ((uint32_t)tid < in_bin) {
      const uint32_t kt = ckey[tid];
      const int ct = cslot[tid];
      uint32_t rank = 0;
      for (uint32_t j0 = 0; j0 < in_bin; j0 += 8) {  // 8 loads per LDS round trip
        uint32_t k2[8];
        int c2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          k2[i] = ckey[j0 + i];  // slots past in_bin (< kWaves * kMaxCand) are ignored
          c2[i] = cslot[j0 + i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          rank += (j0 + i < in_bin && (k2[i] > kt || (k2[i] == kt && c2[i] < ct))) ? 1u : 0u;
      }
      if (rank < remaining) atomicOr(&sh.kbits[ct >> 5], 1u << (ct & 31));
    }
    __syncthreads();
    keep |= (sh.kbits[c0 >> 5] >> (c0 & 31)) & ((1u << KPT) - 1u);
  }
  // ascending ids: a kept block's position is its rank in candidate order.
  // The window's candidates [w0, n) are all kept and come last, so they are
  // written cooperatively; each thread writes its other kept candidates (a
  // few) in a loop over their bits.
  uint32_t total;
  const uint32_t rest = keep & ~in_window;
  const uint32_t at = wg_excl_scan((uint32_t)__popc(rest), sh.scan_tot[2], &total);
  const int n_win = max(0, n - max(w0, 0));  // window candidates present
  const uint32_t cap = (uint32_t)p.out_cap;
  uint32_t pos = at;
  for (uint32_t bits = rest; bits != 0; bits &= bits - 1, ++pos)
    if (pos < cap) list[pos] = c0 + __builtin_ctz(bits);
  for (int i = tid; i < n_win; i += kThreads)
    if (total + (uint32_t)i < cap) list[total + i] = w0 + i;
  total += (uint32_t)n_win;
  const int cnt = (int)min(total, cap);
  __syncthreads();  // the list is complete; scan slots may be reused
  if (gids)
    for (int i = tid; i < cnt; i += kThreads) gids[i] = list[i];
  if (gcnt && tid == 0) *gcnt = cnt;
  return cnt;
}

// Token level with at most kThreads * kTokKeys candidate slots and at most
// kGammaLds selected blocks ("SparDA" article, section 2.3: a finer pass
// keeps single tokens inside the chosen blocks). Slot c is token gamma[c / S] * S + c % S of the unit's block list
// (S = p.ratio); the list is ascending, so slot order is token order. Kept:
// the first min(k, #candidates) candidates by (score desc, slot asc), plus
// every token of the window [T - W, T), candidate or not. Thread t owns
// slots 32t .. 32t + 31, so its keep decisions are the bits of one word and
// the ascending output is one workgroup scan: the kept candidates below the
// window in slot order, then the window's tokens. No bitmap over the
// sequence is needed. Writes the ids and the count to gids / gcnt.
constexpr int kTokKeys = 32;
static_assert(kThreads * kTokKeys / 32 <= kThreads * kRegKeys,
              "ranked-kept bits fit the transposition array");
static_assert(kTokKeys == 32, "one word of keep bits per thread");

__device__ __forceinline__ void topk_tokens(const SelectParams& p, int unit, const UnitGeom& ug,
                                            TopkShared& sh, int32_t* gids, int32_t* gcnt) {
  constexpr int KPT = kTokKeys;
  constexpr int HALF = kThreads * KPT / 2;  // slots transposed per round
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = ug.n, S = p.ratio, T = ug.T;
  const int c0 = KPT * tid;  // first slot of this thread
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring
  float v[KPT];
  uint32_t kmax = 0, kmin_inv = 0;
  {
    // One round trip: coalesced score loads (thread t: slots u * 256 + t),
    // every chunk's key range and the block list, all bounded by the
    // capacities rather than the unit's counts (applied below), so that
    // none of them waits for the count's load. Chunks past the unit's slots
    // published empty ranges; slots past them are masked below.
    const int nmax = p.n_slots_max;
#pragma unroll
    for (int u = 0; u < KPT; ++u) v[u] = published(&sc[min(u * kThreads + tid, nmax - 1)]);
    const int nch = select_chunks(nmax);
    const int32_t* ck = reinterpret_cast<const int32_t*>(p.chunk_keys + (int64_t)unit * nch * 2);
    for (int ch = tid; ch < nch; ch += kThreads) {
      kmax = max(kmax, (uint32_t)published_i32(&ck[2 * ch]));
      kmin_inv = max(kmin_inv, (uint32_t)published_i32(&ck[2 * ch + 1]));
    }
    // the block list, staged in LDS for the token ids of the emission
    for (int i = tid; i < p.gamma_cap; i += kThreads) sh.gam[i] = ug.slots.gamma[i];
    kmax = wave_max_u(kmax);
    kmin_inv = wave_max_u(kmin_inv);
    if (lane == 0) {
      sh.red[1][wave] = kmax;
      sh.red[2][wave] = kmin_inv;
    }
  }
  for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
  if (tid == 0) sh.n_cand = 0u;
  // transposition to the contiguous ownership, HALF slots per round: the
  // threads of half h own slots [h * HALF, (h + 1) * HALF)
  // (keys: 0 = no candidate)
  uint32_t kr[KPT];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h) __syncthreads();  // the first round has been read
#pragma unroll
    for (int u = 0; u < KPT / 2; ++u) sh.xpose[u * kThreads + tid] = v[h * KPT / 2 + u];
    __syncthreads();
    if (tid / (kThreads / 2) == h) {
#pragma unroll
      for (int u = 0; u < KPT; u += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&sh.xpose[c0 - h * HALF + u]);
        kr[u] = order_key(x.x);
        kr[u + 1] = order_key(x.y);
        kr[u + 2] = order_key(x.z);
        kr[u + 3] = order_key(x.w);
      }
    }
  }
  uint32_t present = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    kr[u] = c0 + u < n ? kr[u] : 0u;
    present |= (kr[u] != 0 ? 1u : 0u) << u;
  }
  const uint32_t cnt = wave_sum_u((uint32_t)__popc(present));
  if (lane == 0) sh.red[0][wave] = cnt;
  __syncthreads();  // key counts and ranges; the transposition array is free
  uint32_t* rbits = reinterpret_cast<uint32_t*>(sh.xpose);  // ranked-kept bits, word t: thread t
  rbits[tid] = 0u;
  uint32_t n_valid = 0;
  kmax = 0;
  kmin_inv = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    n_valid += sh.red[0][w2];
    kmax = max(kmax, sh.red[1][w2]);
    kmin_inv = max(kmin_inv, sh.red[2][w2]);
  }
  const uint32_t kmin = ~kmin_inv;
  const uint32_t k_eff = min((uint32_t)max(unit_top_k(p, ug.nb), 0), n_valid);
  const bool keep_all = k_eff > 0 && k_eff == n_valid;
  uint32_t keep = keep_all ? present : 0u;
  uint32_t cand = 0, remaining = 0, in_bin = 0;  // the threshold bucket's candidates to settle
  int mode = 0;                                  // 1: all equal, 2: rank (uniform)
  if (k_eff > 0 && !keep_all) {                  // uniform
    const Threshold th = bucket_threshold<KPT>(sh, kr, present, k_eff, n_valid, kmin, kmax);
    keep = th.keep;
    cand = th.cand;
    remaining = th.remaining;
    in_bin = th.in_bin;
    mode = th.mode;
  }
  if (mode == 1) {
    // every candidate left has the same key: the first `remaining` in slot order
    uint32_t m;
    uint32_t pos = wg_excl_scan((uint32_t)__popc(cand), sh.scan_tot[1], &m);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if ((cand >> u) & 1u) keep |= (pos++ < remaining ? 1u : 0u) << u;
  } else if (mode == 2) {
    // at most kMaxCand candidates: gathered (any order), each ranked against
    // all of them (key desc, slot asc); those ranked below `remaining` are kept
    uint32_t* ckey = &sh.cand_key[0][0];
    int32_t* cslot = &sh.cand_slot[0][0];
    for (uint32_t bits = cand; bits != 0; bits &= bits - 1) {
      const int u = __builtin_ctz(bits);
      uint32_t k = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) k = i == u ? kr[i] : k;
      const uint32_t slot = atomicAdd(&sh.n_cand, 1u);
      ckey[slot] = k;
      cslot[slot] = c0 + u;
    }
    __syncthreads();
    if ((uint32_t)tid < in_bin) {
      const uint32_t kt = ckey[tid];
      const int ct = cslot[tid];
      uint32_t rank = 0;
      for (uint32_t j0 = 0; j0 < in_bin; j0 += 8) {  // 8 loads per LDS round trip
        uint32_t k2[8];
        int c2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          k2[i] = ckey[j0 + i];  // slots past in_bin (< kWaves * kMaxCand) are ignored
          c2[i] = cslot[j0 + i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          rank += (j0 + i < in_bin && (k2[i] > kt || (k2[i] == kt && c2[i] < ct))) ? 1u : 0u;
      }
      if (rank < remaining) atomicOr(&rbits[ct >> 5], 1u << (ct & 31));
    }
    __syncthreads();
    keep |= rbits[tid];
  }
  // emission: kept candidates below the window in slot order, then the
  // window's tokens [lo, T)
  const int lo = p.window > 0 ? max(T - p.window, 0) : T;
  // Slot c0 + u is token e * S + r with (e, r) = (e0, r0 + u) while
  // r0 + u < S, else (e1, r0 + u - S) when S >= KPT (a thread's slots span
  // at most two blocks); smaller S steps through the staged list.
  // (Tokens of slots that hold none are computed but never stored.)
  const int gi0 = c0 / S, r0 = c0 - gi0 * S, gmax = p.gamma_cap - 1;
  const uint32_t e0 = (uint32_t)sh.gam[min(gi0, gmax)], e1 = (uint32_t)sh.gam[min(gi0 + 1, gmax)];
  auto token_of = [&](int u) -> int {
    if (S >= KPT) {  // uniform
      const int r = r0 + u;
      return (int)((r < S ? e0 : e1) * (uint32_t)S + (uint32_t)(r < S ? r : r - S));
    }
    const int q = (r0 + u) / S;
    return (int)((uint32_t)sh.gam[min(gi0 + q, gmax)] * (uint32_t)S + (uint32_t)(r0 + u - q * S));
  };
  // bits u >= x (x clamped to [0, 32])
  auto from_bit = [](int64_t x) -> uint32_t {
    return x <= 0 ? 0xFFFFFFFFu : (x >= 32 ? 0u : 0xFFFFFFFFu << (int)x);
  };
  uint32_t in_window = 0;
  if (S >= KPT) {  // uniform: two runs of consecutive tokens
    const int64_t split = S - r0;  // first u in block e1
    in_window = (from_bit(lo - ((int64_t)e0 * S + r0)) & ~from_bit(split)) |
                (from_bit(split) & from_bit(split + lo - (int64_t)e1 * S));
  } else {
#pragma unroll
    for (int u = 0; u < KPT; ++u) in_window |= (token_of(u) >= lo ? 1u : 0u) << u;
  }
  const uint32_t rest = keep & ~in_window;
  uint32_t total;
  const uint32_t at = wg_excl_scan((uint32_t)__popc(rest), sh.scan_tot[2], &total);
  const uint32_t cap = (uint32_t)p.out_cap;
  // The kept candidates below the window take positions [0, n_rest): written
  // to LDS (the transposition array, free since the scan's barrier) and copied
  // out with coalesced stores when they fit there, else stored directly.
  // Position of kept slot u: at + the kept slots before it (no loop-carried
  // state, so the 32 writes are independent predicated instructions).
  const uint32_t n_rest = min(total, cap);
  auto store_all = [&](int32_t* out, auto&& tok) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const uint32_t pos = at + (uint32_t)__popc(rest & ((1u << u) - 1u));
      if (((rest >> u) & 1u) && pos < cap) out[pos] = tok(u);
    }
  };
  auto token_two = [&](int u) {  // S >= KPT: the slot's block is e0 or e1
    const int r = r0 + u;
    return (int)((r < S ? e0 : e1) * (uint32_t)S + (uint32_t)(r < S ? r : r - S));
  };
  if (n_rest <= (uint32_t)(kThreads * kRegKeys)) {  // uniform
    int32_t* stage = reinterpret_cast<int32_t*>(sh.xpose);
    if (S >= KPT) store_all(stage, token_two);  // uniform
    else store_all(stage, token_of);
    __syncthreads();
    for (uint32_t i = tid; i < n_rest; i += kThreads) gids[i] = stage[i];
  } else {
    if (S >= KPT) store_all(gids, token_two);  // uniform
    else store_all(gids, token_of);
  }
  const int n_win = T - lo;
  for (int i = tid; i < n_win; i += kThreads)
    if (total + (uint32_t)i < cap) gids[total + i] = lo + i;
  if (tid == 0) *gcnt = (int)min(total + (uint32_t)n_win, cap);
}

// Top-k of a unit whose candidates fit in registers (n <= kThreads * kRegKeys):
// thread t keeps the keys of candidates c = u * kThreads + t (u < kRegKeys),
// so the published scores are read with coalesced loads and the histogram
// passes touch LDS only for the histogram. TWO: candidate slots map to fine
// blocks through the kept coarse blocks (else slot c is block c). Sets the
// kept blocks in `bitmap` (zeroed by the caller); every path has a barrier
// before its first mark.
template <bool TWO>
__device__ __forceinline__ void topk_regs(const SelectParams& p, int unit, const UnitGeom& ug,
                                          TopkShared& sh, uint32_t* bitmap) {
  constexpr int KPT = kRegKeys;
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = ug.n;
  // Score loads (coalesced) and the coarse entries bounded by the
  // capacities, so that they do not wait for the unit's counts; slots past
  // n are masked below.
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring
  float v[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u)  // unconditional (clamped), coalesced loads that overlap
    v[u] = published(&sc[min(u * kThreads + tid, p.n_slots_max - 1)]);
  // the block of each of this thread's candidates (-1: none). TWO: slot c is
  // offset c % ratio of coarse entry c / ratio; quotient and remainder are
  // stepped from candidate to candidate (no division each).
  int blk[KPT];
  int ent[KPT], gis[KPT], off[KPT];
  if (TWO) {
    const int ratio = p.ratio;
    const int dq = kThreads / ratio, dr = kThreads - dq * ratio;
    int gi = tid / ratio, r = tid - gi * ratio;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      gis[u] = gi;
      off[u] = r;
      ent[u] = ug.slots.gamma[min(gi, p.gamma_cap - 1)];
      gi += dq;
      r += dr;
      if (r >= ratio) {
        r -= ratio;
        ++gi;
      }
    }
  }
  if (n <= 0) {  // uniform
    __syncthreads();
    return;
  }
  if (TWO) {
    const int gc = ug.slots.gcnt;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      blk[u] = u * kThreads + tid < n && gis[u] < gc ? ug.slots.from_entry(ent[u], off[u]) : -1;
  } else {
#pragma unroll
    for (int u = 0; u < KPT; ++u) blk[u] = u * kThreads + tid < n ? u * kThreads + tid : -1;
  }
  // the first histogram is cleared while the loads are in flight
  for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
  uint32_t kr[KPT];
  uint32_t cnt = 0, kmax = 0, kmin_inv = 0;  // kmin_inv: largest ~key
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const bool ok = blk[u] >= 0;
    const uint32_t k = ok ? order_key(v[u]) : 0u;
    kr[u] = k;
    kmax = max(kmax, k);
    kmin_inv = max(kmin_inv, ok ? ~k : 0u);
    if (TWO) cnt += ok ? 1u : 0u;
  }
  kmax = wave_max_u(kmax);
  kmin_inv = wave_max_u(kmin_inv);
  if (TWO) cnt = wave_sum_u(cnt);
  if (lane == 0) {
    sh.red[0][wave] = cnt;
    sh.red[1][wave] = kmax;
    sh.red[2][wave] = kmin_inv;
  }
  __syncthreads();
  uint32_t n_valid = TWO ? 0u : (uint32_t)n;
  kmax = 0;
  kmin_inv = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (TWO) n_valid += sh.red[0][w];
    kmax = max(kmax, sh.red[1][w]);
    kmin_inv = max(kmin_inv, sh.red[2][w]);
  }
  const uint32_t kmin = ~kmin_inv;
  const uint32_t k_eff = min((uint32_t)max(unit_top_k(p, ug.nb), 0), n_valid);
  if (k_eff == 0) return;
  if (k_eff == n_valid) {  // every candidate is kept
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (kr[u]) mark(bitmap, blk[u]);
    return;
  }
  uint32_t present = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) present |= (blk[u] >= 0 ? 1u : 0u) << u;
  const Threshold th = bucket_threshold<KPT>(sh, kr, present, k_eff, n_valid, kmin, kmax);
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if ((th.keep >> u) & 1u) mark(bitmap, blk[u]);
  const uint32_t remaining = th.remaining;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  if (th.mode == 2) {  // uniform
    // at most kMaxCand keys left: gathered per wave with ballots, each ranked
    // against all of them (key desc, candidate asc)
    uint32_t wrun = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool inb = (th.cand >> u) & 1u;
      const uint64_t m = __ballot(inb);
      if (inb) {
        const uint32_t pos = wrun + (uint32_t)__popcll(m & below);
        sh.cand_key[wave][pos] = kr[u];
        sh.cand_slot[wave][pos] = u * kThreads + tid;
        sh.cand_blk[wave][pos] = blk[u];
      }
      wrun += (uint32_t)__popcll(m);
    }
    if (lane == 0) sh.wcnt[wave] = wrun;
    __syncthreads();
    uint32_t wc[kWaves], first = 0;
    int w = -1;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      wc[w2] = sh.wcnt[w2];
      if (w < 0 && (uint32_t)tid < first + wc[w2]) w = w2;
      if (w < 0) first += wc[w2];
    }
    if (w >= 0) {
      const uint32_t kt = sh.cand_key[w][tid - first];
      const int ct = sh.cand_slot[w][tid - first], bt = sh.cand_blk[w][tid - first];
      uint32_t rank = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2)
        for (uint32_t j0 = 0; j0 < wc[w2]; j0 += 8) {  // 8 loads per LDS round trip
          uint32_t k2[8];
          int c2[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {  // j0 + i < kMaxCand (a multiple of 8); later ones ignored
            k2[i] = sh.cand_key[w2][j0 + i];
            c2[i] = sh.cand_slot[w2][j0 + i];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i)
            rank += (j0 + i < wc[w2] && (k2[i] > kt || (k2[i] == kt && c2[i] < ct))) ? 1u : 0u;
        }
      if (rank < remaining) mark(bitmap, bt);
    }
  } else if (th.mode == 1) {  // uniform
    // more than kMaxCand keys, all equal: the first `remaining` of them in
    // candidate order are kept. Rank of a tie = ties at earlier slots, then
    // at earlier waves of the same slot, then at lower lanes.
    uint64_t tie_mask[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      tie_mask[u] = __ballot((th.cand >> u) & 1u);
      if (lane == 0) sh.tie_cnt[u][wave] = (uint32_t)__popcll(tie_mask[u]);
    }
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      uint32_t in_slot = 0, waves_before = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const uint32_t cw = sh.tie_cnt[u][w2];
        in_slot += cw;
        waves_before += w2 < wave ? cw : 0u;
      }
      if (((th.cand >> u) & 1u) &&
          before + waves_before + (uint32_t)__popcll(tie_mask[u] & below) < remaining)
        mark(bitmap, blk[u]);
      before += in_slot;
    }
  }
}

// Top-k of a unit with more candidates than the register path holds: keys in
// LDS (`sk`, when lds_keys) or re-read from the published scores; full 11-bit
// radix passes down to the exact threshold, ties ranked by a scan in
// candidate order. Sets the kept blocks in `bitmap` (zeroed by the caller).
__device__ __forceinline__ void topk_general(const SelectParams& p, int unit, const UnitGeom& ug,
                                             TopkShared& sh, uint32_t* bitmap, uint32_t* sk,
                                             bool lds_keys) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = ug.n;
  const SlotMap& slots = ug.slots;
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring

  // 1. keys (0 = not a candidate), their number, largest and smallest key;
  //    the published scores are loaded in unrolled batches so they overlap
  uint32_t cnt = 0, kmax = 0, kmin = 0xFFFFFFFFu;
  constexpr int kBatch = 16;
  for (int cb = 0; cb < n; cb += kThreads * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = cb + u * kThreads + tid;  // unconditional (clamped) loads overlap
      v[u] = published(&sc[min(c, n - 1)]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = cb + u * kThreads + tid;
      const uint32_t k = c < n ? order_key(v[u]) : 0u;  // 0 for kAbsentScore slots
      if (lds_keys && c < n) sk[c] = k;
      if (k) {
        ++cnt;
        kmax = max(kmax, k);
        kmin = min(kmin, k);
      }
    }
  }
  cnt = wave_sum_u(cnt);
  kmax = wave_max_u(kmax);
  kmin = wave_min_u(kmin);
  if (lane == 0) {
    sh.red[0][wave] = cnt;
    sh.red[1][wave] = kmax;
    sh.red[2][wave] = kmin;
  }
  __syncthreads();
  uint32_t n_valid = 0;
  kmax = 0;
  kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    n_valid += sh.red[0][w];
    kmax = max(kmax, sh.red[1][w]);
    kmin = min(kmin, sh.red[2][w]);
  }
  auto key_of = [&](int c) -> uint32_t {
    if (lds_keys) return sk[c];
    return order_key(published(&sc[c]));
  };
  const uint32_t k_eff = min((uint32_t)max(unit_top_k(p, ug.nb), 0), n_valid);
  if (k_eff == 0) return;
  const bool keep_all = k_eff == n_valid;

  // 2. the k-th largest key `thr` and how many keys equal to it are kept
  uint32_t thr = 0, ties_keep = 0;
  if (!keep_all && kmax == kmin) {
    thr = kmax;
    ties_keep = k_eff;
  } else if (!keep_all) {
    const int common = __clz(kmax ^ kmin);  // < 32 here
    int shift = 32 - common;
    uint32_t prefix = common == 0 ? 0u : (kmax & ~(0xFFFFFFFFu >> common));
    uint32_t remaining = k_eff;
    while (shift > 0) {
      const int db = shift < kDigitBits ? shift : kDigitBits;
      shift -= db;
      const int hi = shift + db;  // bits at and above `hi` must equal the prefix
      const int nbins = 1 << db;
      for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
      __syncthreads();
      // branch-free: a key outside the current prefix (or absent) counts in
      // the lane's dummy bin; four keys per iteration
      const uint32_t hmask = (uint32_t)((uint64_t)0xFFFFFFFFu << hi);  // bits at and above hi
      const uint32_t dummy = kBins + (tid & (kWave - 1));
      for (int c = tid; c < n; c += 4 * kThreads) {
        uint32_t k4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) k4[i] = c + i * kThreads < n ? key_of(c + i * kThreads) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool in = k4[i] != 0u && ((k4[i] ^ prefix) & hmask) == 0u;
          atomicAdd(&sh.hist[in ? hist_slot((k4[i] >> shift) & (uint32_t)(nbins - 1)) : dummy], 1u);
        }
      }
      __syncthreads();
      take_digit(sh, nbins, shift, prefix, remaining);
    }
    thr = prefix;
    ties_keep = remaining;
  }

  // 3. mark kept blocks; thread t scans candidates [t*per, (t+1)*per) in order
  const int per = (n + kThreads - 1) / kThreads;
  const int c0 = tid * per, c1 = min(c0 + per, n);
  // the first two coarse entries of the thread's run, loaded before the tie
  // count so that their latency overlaps it
  const bool two = slots.gamma != nullptr;
  int gi = two ? c0 / slots.ratio : 0, r = two ? c0 - gi * slots.ratio : 0;
  const int gi0 = gi;
  const int pre0 = two && gi0 < slots.gcnt ? slots.gamma[gi0] : -1;
  const int pre1 = two && gi0 + 1 < slots.gcnt ? slots.gamma[gi0 + 1] : -1;
  uint32_t ties = 0;
  if (!keep_all)
    for (int c = c0; c < c1; ++c) ties += key_of(c) == thr ? 1u : 0u;
  uint32_t tot;
  uint32_t rank = block_excl_scan(ties, &tot, sh);
  // consecutive candidates share their coarse entry (ratio slots each): its
  // id is loaded once per entry, and the entry and the offset in it advance
  // with the candidate instead of being divided out of it
  int last_gi = -1, last_base = -1;
  for (int c = c0; c < c1; ++c) {
    const uint32_t k = key_of(c);
    bool keep = k != 0u && (keep_all || k > thr);
    if (k != 0u && !keep && k == thr) keep = rank++ < ties_keep;
    if (keep) {
      int beta;
      if (!two) {
        beta = c < slots.nb ? c : -1;
      } else {
        if (gi != last_gi) {
          last_gi = gi;
          const int gg = gi == gi0       ? pre0
                         : gi == gi0 + 1 ? pre1
                                         : (gi < slots.gcnt ? slots.gamma[gi] : -1);
          last_base = gg >= 0 ? gg * slots.ratio : -1;
        }
        beta = last_base < 0 ? -1 : last_base + r;
        beta = beta < slots.nb ? beta : -1;
      }
      if (beta >= 0) mark(bitmap, beta);
    }
    if (two && ++r == slots.ratio) {
      r = 0;
      ++gi;
    }
  }
}

// Window and caller-forced blocks into the bitmap, then the bitmap as
// ascending ids: to `list` (LDS, out_cap + kWave entries, the last kWave a
// scratch area) and, if not null, to `gids` / `*gcnt` (global). Wave w emits its quarter of the bitmap words, 64 words per
// round: lane l takes one word, a wave prefix sum of the words' popcounts
// gives each its first position, and the lane writes its set bits in order.
// Returns the count in every thread; the list is complete when it returns.
__device__ __forceinline__ int emit_ids(const SelectParams& p, int unit, const UnitGeom& ug,
                                        uint32_t* bitmap,
                                        TopkShared& sh, int32_t* list, int32_t* gids,
                                        int32_t* gcnt) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int S = p.block_size, nb = ug.nb;
  const int words = (nb + 31) / 32;
  if (p.window > 0) {
    const int64_t lo_tok = (int64_t)ug.T - p.window;
    const int w0 = lo_tok <= 0 ? 0 : (int)(lo_tok / S);
    for (int beta = w0 + tid; beta < nb; beta += kThreads) mark(bitmap, beta);
  }
  if (p.forced) {  // caller-forced blocks
    const int32_t* forced = p.forced + (int64_t)unit * p.forced_cap;
    for (int i = tid; i < p.forced_cap; i += kThreads) {
      const int f = forced[i];
      if (f >= 0 && f < nb) mark(bitmap, f);
    }
  }
  __syncthreads();
  const int wpw = (words + kWaves - 1) / kWaves;  // words of each wave
  const int w_lo = wave * wpw, w_hi = min(w_lo + wpw, words);
  // The wave's non-zero words (index, bits) are compacted, in order, into its
  // share of sh.xpose (free once the top-k is done), so the bit loop below
  // runs over them only: a sparse bitmap (a token level marks ~1.5 K bits of
  // 131 K) would otherwise cost a round per 64 words whatever they hold.
  constexpr int kScrWords = kThreads * kRegKeys / kWaves / 2;  // pairs per wave
  uint32_t* scr_idx = reinterpret_cast<uint32_t*>(sh.xpose) + wave * 2 * kScrWords;
  uint32_t* scr_bits = scr_idx + kScrWords;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t ones = 0, nz = 0;  // nz: the wave's non-zero words so far (uniform)
  for (int wb = w_lo; wb < w_hi; wb += kWave) {  // wave-uniform
    const int w = wb + lane;
    const uint32_t x = w < w_hi ? bitmap[w] : 0u;
    ones += __popc(x);
    const uint64_t m = __ballot(x != 0u);
    const uint32_t at = nz + (uint32_t)__popcll(m & below);
    if (x != 0u && at < (uint32_t)kScrWords) {
      scr_idx[at] = (uint32_t)w;
      scr_bits[at] = x;
    }
    nz += (uint32_t)__popcll(m);
  }
  const bool compact = nz <= (uint32_t)kScrWords;  // else the full scan below
  ones = wave_sum_u(ones);
  if (lane == 0) sh.wave_tot[wave] = ones;
  __syncthreads();
  uint32_t pos = 0, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    const uint32_t t = sh.wave_tot[w2];
    pos += w2 < wave ? t : 0u;
    total += t;
  }
  // The bit loop has a wave-uniform trip count (the wave's largest popcount)
  // and no branch: a lane without a bit left, or past the capacity, writes
  // its trash slot list[cap + lane]. The global copy follows, coalesced.
  const uint32_t cap = (uint32_t)p.out_cap;
  const uint32_t trash = cap + (uint32_t)lane;
  const int r_end = compact ? (int)nz : w_hi - w_lo;
  for (int rb = 0; rb < r_end; rb += kWave) {  // wave-uniform: 64 words per round
    const int j = rb + lane;
    int w;
    uint32_t x;
    if (compact) {
      w = j < r_end ? (int)scr_idx[j] : 0;
      x = j < r_end ? scr_bits[j] : 0u;
    } else {
      w = w_lo + j;
      x = j < r_end ? bitmap[w] : 0u;
    }
    const uint32_t c = (uint32_t)__popc(x);
    const uint32_t incl = wave_incl_scan(c);
    uint32_t at = pos + incl - c;
    const int iters = (int)wave_max_u(c);
    for (int i = 0; i < iters; ++i) {
      const bool has = x != 0u;
      list[has && at < cap ? at : trash] = w * 32 + __builtin_ctz(x | 0x80000000u);
      x &= x - 1u;
      at += has ? 1u : 0u;
    }
    pos += (uint32_t)__shfl((int)incl, kWave - 1);
  }
  const int cnt = (int)min(total, cap);
  if (gcnt && tid == 0) *gcnt = cnt;
  __syncthreads();
  if (gids)
    for (int i = tid; i < cnt; i += kThreads) gids[i] = list[i];
  return cnt;
}

// The whole selection of one unit by one workgroup, from the published
// scores: top-k, window, ascending ids. ug = unit_geom(p, unit) (callers
// compute it early so its loads overlap other work). dyn = dynamic LDS laid
// out as [bitmap: out_blocks_max bits][keys: n_slots_max words, general path].
// list: the ids in LDS (out_cap + kWave entries, never null); gids / gcnt:
// their global copy and count, or null.
__device__ __forceinline__ int select_from_scores(const SelectParams& p, int unit,
                                                  const UnitGeom& ug, TopkShared& sh,
                                                  uint32_t* dyn, int32_t* list, int32_t* gids,
                                                  int32_t* gcnt) {
  // The path and the bitmap's extent follow the capacities, not the unit's
  // counts, so that the score loads do not wait for the counts' loads.
  if (!p.gamma && p.n_slots_max <= kThreads * kRegKeys)
    return topk_single(p, unit, ug, sh, list, gids, gcnt);
  uint32_t* bitmap = dyn;
  for (int w = thread_id(); w < (p.out_blocks_max + 31) / 32; w += kThreads) bitmap[w] = 0u;
  if (p.gamma && p.n_slots_max <= kThreads * kRegKeys) {
    topk_regs<true>(p, unit, ug, sh, bitmap);
  } else {
    __syncthreads();
    uint32_t* sk = dyn + (p.out_blocks_max + 31) / 32;
    topk_general(p, unit, ug, sh, bitmap, sk, p.n_slots_max <= kLdsKeys);
  }
  return emit_ids(p, unit, ug, bitmap, sh, list, gids, gcnt);
}

// One scoring task: rows [chunk * kRowsPerWG, (chunk + 1) * kRowsPerWG) of
// the unit's candidate slots, by the whole workgroup; their scores are
// published (device-coherent stores) when it returns. With
// p.refresh_begin >= 0 (single level) the chunk's blocks at or beyond it are
// first rebuilt from the K cache and stored (the per-step refresh of the
// growing block), then scored from the stored rows with the same arithmetic
// as every other row.
// TS: storage type of a summary element (float for mean rows, TE for boxes).
// UNR: rows in flight per lane group (kUnroll, or more where registers allow).
template <typename TE, int D, int KIND, int G, int UNR = kUnroll>
__device__ __forceinline__ void score_chunk(const SelectParams& p, int unit, int chunk,
                                            TopkShared& sh) {
  constexpr bool kTok = KIND == kKindTokens;  // rows are token K rows (page table)
  using TS = typename std::conditional<KIND == HS_SUMMARY_MEAN, float, TE>::type;
  constexpr int EPS = 16 / sizeof(TS);                        // elements per 16-byte load
  constexpr int ROW = (KIND == HS_SUMMARY_MINMAX ? 2 : 1) * D;  // elements per row
  constexpr int LPR = ROW / EPS;                              // lanes per row
  constexpr int RPW = kWave / LPR;                            // rows per wave instruction
  constexpr int64_t kRowBytes = ROW * sizeof(TS);
  const KvView& kv = p.kv;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const UnitGeom ug = unit_geom(p, unit);
  const int n_slots = ug.n;
  const int c_wg = chunk * kRowsPerWG;  // first slot of the workgroup
  const int c_begin = c_wg + wave * kRowsPerWave;
  const int li = lane % LPR, rg = lane / LPR;
  static_assert(kRowsPerWG <= kThreads, "at most one staged score per thread");
  static_assert(kRowsPerWG <= kGammaLds, "a chunk's coarse entries fit the staging array");
  if constexpr (kTok) {  // a staged row that holds no token keeps the absent score
    if (tid < kRowsPerWG) sh.stage[tid] = __uint_as_float(kAbsentScore);
  }
  // Slots map to blocks through coarse entries (two levels, token level):
  // the chunk's entries [g_lo, g_hi) are staged in LDS first (their loads
  // overlap the query loads below), so that no row load waits on a lookup.
  // The staged range is bounded by the list's capacity, not its count, so
  // these loads do not wait for the count's.
  const bool via_gamma = ug.slots.gamma != nullptr;  // uniform
  const int g_lo = via_gamma ? c_wg / p.ratio : 0;
  const int g_cap = via_gamma ? min((c_wg + kRowsPerWG - 1) / p.ratio + 1, p.gamma_cap) : 0;
  const int g_hi = via_gamma ? min(g_cap, ug.slots.gcnt) : 0;
  for (int i = tid; i < g_cap - g_lo; i += kThreads) sh.gam[i] = ug.slots.gamma[g_lo + i];
  auto block_of = [&](int c) {
    if (!via_gamma) return ug.slots.block_of(c);
    const int gi = c / p.ratio;
    return gi < g_hi ? ug.slots.from_entry(sh.gam[gi - g_lo], c - gi * p.ratio) : -1;
  };

  // the unit's G query heads folded into per-element coefficients
  float coef[EPS];
  {
    const int e0 = li * EPS;                                // first element of the lane
    const int part = KIND == HS_SUMMARY_MINMAX ? e0 / D : 0;  // 0: min (mean, token), 1: max
    const int dim0 = e0 % D;
#pragma unroll
    for (int k = 0; k < EPS; ++k) {
      float c = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float qv = load_elem<TE>(
            p.q, ((int64_t)b * kv.num_kv_heads * G + g * G + j) * D + dim0 + k);
        if (KIND != HS_SUMMARY_MINMAX) c += qv;
        else c += part == 0 ? fminf(qv, 0.f) : fmaxf(qv, 0.f);
      }
      coef[k] = c;
    }
  }
  if (via_gamma || kTok) __syncthreads();  // staged coarse entries, absent scores of token rows
  // score of one row from the EPS elements each of its LPR lanes holds
  auto row_dot = [&](const float (&f)[EPS]) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < EPS; ++k) acc = fmaf(coef[k], f[k], acc);
    return group_sum<LPR>(acc);
  };
  auto row_score = [&](const uint4& r) {
    float f[EPS];
    Vec16<TS>::unpack(r, f);
    return row_dot(f);
  };
  // Refresh of this chunk's blocks in [refresh_begin, n): when each such
  // block has a wave of its own and few enough tokens, the wave issues the
  // block's K loads before the streaming loop below and rebuilds, stores and
  // scores the row (from registers, with the stored values) after it.
  constexpr int kRefreshLoads = 16;
  constexpr int kTPW = kWave / (D / Vec16<TE>::EPL);  // tokens per K load instruction
  const int r0 = max(p.refresh_begin, c_wg), r1 = min(n_slots, c_wg + kRowsPerWG);
  const bool refresh = !kTok && p.refresh_begin >= 0 && p.gamma == nullptr && r0 < r1;  // uniform
  const bool early = refresh && p.rebuilt_by == nullptr && r1 - r0 <= kWaves &&
                     p.block_size <= kRefreshLoads * kTPW;
  const int my_row = r0 + wave;
  uint4 rk[kRefreshLoads];
  uint32_t rk_ok = 0;
  if constexpr (!kTok)
    if (early && my_row < r1) rk_ok = summ_load<TE, D, kRefreshLoads>(kv, b, g, my_row, p.block_size, ug.T, rk);
  const uint8_t* summ = reinterpret_cast<const uint8_t*>(p.summ) +
                        (int64_t)unit * p.max_blocks * kRowBytes;
  if (c_begin < n_slots) {  // wave-uniform
    const int c_end = min(c_begin + kRowsPerWave, n_slots);
    static_assert(UNR <= 32, "one bit per row in flight");
    for (int cb = c_begin; cb < c_end; cb += RPW * UNR) {
      uint4 r[UNR];
      uint32_t ok = 0;  // bit u: row cb + u * RPW + rg holds a candidate
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = cb + u * RPW + rg;
        if constexpr (kTok) {
          // slot -> token through the staged block list, then its page
          const int beta = c < c_end ? block_of(c) : -1;
          const int64_t off = beta >= 0 ? row_offset(kv, b, g, beta) : -1;
          ok |= (off >= 0 ? 1u : 0u) << u;
          r[u] = off >= 0 ? *reinterpret_cast<const uint4*>(kv.k_pool + off + li * 16)
                          : make_uint4(0, 0, 0, 0);
        } else {
          const int beta = c < c_end ? block_of(c) : -1;
          ok |= (beta >= 0 ? 1u : 0u) << u;
          r[u] = beta >= 0 ? *reinterpret_cast<const uint4*>(summ + beta * kRowBytes + li * 16)
                           : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float acc = row_score(r[u]);
        if (li == 0 && ((ok >> u) & 1u)) sh.stage[cb + u * RPW + rg - c_wg] = acc;
      }
    }
  }
  if constexpr (!kTok) {  // refresh (summary kinds only)
    if (early) {
      __syncthreads();  // the stale scores of the refreshed rows are staged
      if (my_row < r1) {
        float a0[Vec16<TE>::EPL], a1[Vec16<TE>::EPL];
        summ_reduce<TE, D, KIND, kRefreshLoads>(rk, rk_ok, a0, a1);
        const int n_tok = min(my_row * p.block_size + p.block_size, ug.T) - my_row * p.block_size;
        summ_store<TE, D, KIND>(const_cast<void*>(p.summ), (int64_t)unit * p.max_blocks + my_row,
                                a0, a1, n_tok);
        float f[EPS];
        summ_row_elems<TE, D, KIND, EPS>(a0, a1, n_tok, f);
        const float acc = row_dot(f);
        if (lane == 0) sh.stage[my_row - c_wg] = acc;
      }
    } else if (refresh) {
      // more blocks than waves, or long blocks: rebuild and store (here, or by
      // another workgroup, whose arrival is awaited), then score the stored
      // rows (device-coherent loads)
      if (p.rebuilt_by != nullptr) {
        if (tid == 0) {
          int32_t* w = counter_of(p.rebuilt_by, unit);
          const long long t0 = wall_clock64();
          for (int i = 0; published_i32(w) < 1; ++i) {
            __builtin_amdgcn_s_sleep(2);
            if ((i & 63) == 63 && wall_clock64() - t0 > p.wait_ticks) {
              publish_i32(p.status, HS_STEP_WAIT_EXPIRED);
              break;
            }
          }
          __hip_atomic_fetch_add(w, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        for (int beta = r0 + wave; beta < r1; beta += kWaves)
          summarize_block<TE, D, KIND, 4>(kv, const_cast<void*>(p.summ),
                                       (int64_t)unit * p.max_blocks + beta, b, g, beta,
                                       p.block_size, ug.T);
      }
      __builtin_amdgcn_s_waitcnt(0);  // rebuilt rows are stored
      __syncthreads();                // (and the stale scores of those rows staged)
      for (int cb = r0 + wave * RPW; cb < r1; cb += kWaves * RPW) {  // wave-uniform
        const int c = min(cb + rg, r1 - 1);
        const int32_t* w = reinterpret_cast<const int32_t*>(summ + c * kRowBytes + li * 16);
        const uint4 r = make_uint4(published_i32(w), published_i32(w + 1), published_i32(w + 2),
                                   published_i32(w + 3));
        const float acc = row_score(r);
        if (li == 0 && cb + rg < r1) sh.stage[cb + rg - c_wg] = acc;
      }
    }
  }
  // publish the workgroup's scores with one coalesced store per thread, and
  // the chunk's largest key and largest ~key (its key range for the top-k)
  __syncthreads();
  const int c = c_wg + tid;
  const bool in = tid < kRowsPerWG && c < n_slots;
  bool ok;
  if constexpr (kTok) ok = in && __float_as_uint(sh.stage[tid]) != kAbsentScore;
  else ok = in && block_of(c) >= 0;
  uint32_t kx = 0, ki = 0;
  if (ok) {
    const float v = sh.stage[tid];
    publish(&p.scores[(int64_t)unit * p.n_slots_max + c], v);
    kx = order_key(v);
    ki = ~kx;
  } else if (in) {  // a slot without a candidate: the all-ones NaN, whose key is 0 (absent)
    publish(&p.scores[(int64_t)unit * p.n_slots_max + c], __uint_as_float(kAbsentScore));
  }
  kx = wave_max_u(kx);
  ki = wave_max_u(ki);
  if (lane == 0) {
    sh.red[1][wave] = kx;
    sh.red[2][wave] = ki;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      kx = max(kx, sh.red[1][w]);
      ki = max(ki, sh.red[2][w]);
    }
    uint32_t* ck = p.chunk_keys + ((int64_t)unit * select_chunks(p.n_slots_max) + chunk) * 2;
    publish_i32(reinterpret_cast<int32_t*>(ck), (int32_t)kx);
    publish_i32(reinterpret_cast<int32_t*>(ck + 1), (int32_t)ki);
  }
}

// One task of the selection kernel: score a chunk, arrive on the unit's
// counter (nchunks tasks); the last one to arrive selects and writes the
// unit's ids and count to global memory.
// list: LDS staging of the id list (out_cap + kWave entries).
template <typename TE, int D, int KIND, int G>
__device__ __forceinline__ void select_task(const SelectParams& p, int unit, int chunk, int nchunks,
                                            TopkShared& sh, uint32_t* dyn, int32_t* list) {
  score_chunk<TE, D, KIND, G>(p, unit, chunk, sh);
  if (!arrive_last(counter_of(p.counters, unit), nchunks, &sh.last)) return;
  if constexpr (KIND == kKindTokens) {
    if (p.n_slots_max <= kThreads * kTokKeys && p.gamma_cap <= kGammaLds) {  // uniform
      topk_tokens(p, unit, unit_geom(p, unit), sh, p.out_ids + (int64_t)unit * p.out_cap,
                  p.out_cnt + unit);
      return;
    }
  }
  select_from_scores(p, unit, unit_geom(p, unit), sh, dyn, list,
                     p.out_ids + (int64_t)unit * p.out_cap, p.out_cnt + unit);
}

}  // namespace
}  // namespace hs
