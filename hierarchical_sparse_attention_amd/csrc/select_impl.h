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
//    workspace.
//  * top-k - the unit's last workgroup to finish scoring (arrival counter in
//    the workspace) selects. Exact radix select on order-preserving uint32
//    keys of the fp32 scores: the leading bits shared by every key are
//    skipped, then 11-bit digits are resolved with an LDS histogram until
//    the k-th largest key is known. Keys above it are kept; keys equal to it
//    are kept in ascending candidate order (candidate order is ascending
//    block order), which is the lowest-index tie-break. Kept blocks and the
//    window's blocks are set in an LDS bitmap, written out as ascending ids.
#pragma once

#include <type_traits>

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int kUnroll = 8;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kBins / kThreads;
constexpr int kRegKeys = 16;    // keys per thread of the register path (<= 4096 candidates)
constexpr int kLdsKeys = 8192;  // beyond this many candidates keys stay in the workspace

// slot c -> block id (or -1 if the slot holds no candidate)
struct SlotMap {
  const int32_t* gamma;
  int gcnt, ratio, nb;
  __device__ __forceinline__ int block_of(int c) const {
    if (gamma == nullptr) return c < nb ? c : -1;
    const int gi = c / ratio;
    if (gi >= gcnt) return -1;
    const int beta = gamma[gi] * ratio + c % ratio;
    return beta < nb ? beta : -1;
  }
};

__device__ __forceinline__ SlotMap make_slots(const SelectParams& p, int unit, int nb) {
  SlotMap m;
  m.nb = nb;
  m.ratio = p.ratio;
  m.gamma = nullptr;
  m.gcnt = 0;
  if (p.gamma) {
    int gc = p.gamma_cnt[unit];
    gc = gc < 0 ? 0 : (gc > p.gamma_cap ? p.gamma_cap : gc);
    m.gamma = p.gamma + (int64_t)unit * p.gamma_cap;
    m.gcnt = gc;
  }
  return m;
}

template <typename TE>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (sizeof(TE) == 4) return reinterpret_cast<const float*>(base)[i];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t tie_cnt[kRegKeys][kWaves];
  float stage[kRowsPerWG];                     // scores of this workgroup's rows
  uint32_t wave_tot[kWaves];
  uint32_t red[3][kWaves];
  uint32_t bcast[4];
  int last;
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
// every thread and returns hist[d] (after the last pass: the number of keys
// equal to the threshold).
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

// Window blocks into the bitmap, then the bitmap as ascending ids. Ids and
// count are written with device-coherent stores, so that a workgroup of the
// same launch on another XCD can read them once this one has drained them.
__device__ __forceinline__ void emit_ids(const SelectParams& p, int unit, int T, int nb, uint32_t* bitmap,
                         TopkShared& sh) {
  const int tid = thread_id();
  const int S = p.block_size;
  const int words = (nb + 31) / 32;
  if (p.window > 0) {
    const int64_t lo_tok = (int64_t)T - p.window;
    const int w0 = lo_tok <= 0 ? 0 : (int)(lo_tok / S);
    for (int beta = w0 + tid; beta < nb; beta += kThreads)
      atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
  }
  __syncthreads();
  // thread t owns bitmap words [t*wpt, (t+1)*wpt)
  const int wpt = (words + kThreads - 1) / kThreads;
  const int w0 = tid * wpt, w1 = min(w0 + wpt, words);
  uint32_t ones = 0;
  for (int w = w0; w < w1; ++w) ones += __popc(bitmap[w]);
  uint32_t total;
  uint32_t pos = block_excl_scan(ones, &total, sh);
  int32_t* ids = p.out_ids + (int64_t)unit * p.out_cap;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bitmap[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)p.out_cap) publish_i32(&ids[pos], w * 32 + bit);
      ++pos;
    }
  }
  if (tid == 0) publish_i32(&p.out_cnt[unit], (int32_t)min(total, (uint32_t)p.out_cap));
}

// Fast path for units with at most kThreads * KPT candidates: thread t keeps
// the keys of candidates c = u * kThreads + t (u < KPT) in registers, so the
// published scores are read with coalesced loads and the histogram passes
// touch LDS only for the histogram. Ties at the threshold are ranked in
// ascending candidate order with per-slot wave ballots.
template <int KPT>
__device__ __forceinline__ void select_unit_regs(const SelectParams& p, int unit, int T, const SlotMap& slots,
                                 int n, TopkShared& sh, uint32_t* bitmap) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int nb = slots.nb;
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring
  for (int w = tid; w < (nb + 31) / 32; w += kThreads) bitmap[w] = 0u;
  float v[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u)  // unconditional (clamped), coalesced loads that overlap
    v[u] = published(&sc[min(u * kThreads + tid, n - 1)]);
  uint32_t kr[KPT];
  uint32_t cnt = 0, kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int c = u * kThreads + tid;
    const uint32_t k = (c < n && slots.block_of(c) >= 0) ? order_key(v[u]) : 0u;
    kr[u] = k;
    if (k) {
      ++cnt;
      kmax = max(kmax, k);
      kmin = min(kmin, k);
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
  const uint32_t k_eff = min((uint32_t)max(p.top_k, 0), n_valid);
  const bool keep_none = k_eff == 0;
  bool keep_all = !keep_none && k_eff == n_valid;
  uint32_t thr = 0, ties_keep = 0, ties_total = 0;
  if (!keep_none && !keep_all && kmax == kmin) {
    thr = kmax;
    ties_keep = k_eff;
    ties_total = n_valid;
  } else if (!keep_none && !keep_all) {
    const int common = __clz(kmax ^ kmin);  // < 32 here
    int shift = 32 - common;
    uint32_t prefix = common == 0 ? 0u : (kmax & ~(0xFFFFFFFFu >> common));
    uint32_t remaining = k_eff;
    while (shift > 0) {
      const int db = shift < kDigitBits ? shift : kDigitBits;
      shift -= db;
      const int hi = shift + db;
      const uint32_t dmask = (1u << db) - 1u;
      for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const uint32_t k = kr[u];
        if (k != 0 && (hi >= 32 || (k >> hi) == (prefix >> hi)))
          atomicAdd(&sh.hist[hist_slot((k >> shift) & dmask)], 1u);
      }
      __syncthreads();
      ties_total = take_digit(sh, 1 << db, shift, prefix, remaining);
    }
    thr = prefix;
    ties_keep = remaining;
  }
  // every key equal to the threshold is kept (the usual case): no ranking needed
  const bool all_ties = !keep_none && !keep_all && ties_keep == ties_total;
  if (!keep_none && (keep_all || all_ties)) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const uint32_t k = kr[u];
      if (k != 0 && (keep_all || k >= thr)) {
        const int beta = slots.block_of(u * kThreads + tid);
        atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
      }
    }
    keep_all = true;  // marked; skip the ranking below
  }
  if (!keep_none && !keep_all) {
    // rank of a tie = number of ties at smaller candidate indices: earlier
    // slots, then earlier waves of the same slot, then lower lanes
    uint64_t tie_mask[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      tie_mask[u] = __ballot(!keep_all && kr[u] != 0 && kr[u] == thr);
      if (lane == 0) sh.tie_cnt[u][wave] = (uint32_t)__popcll(tie_mask[u]);
    }
    __syncthreads();
    uint32_t before = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      uint32_t in_slot = 0, waves_before = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t cw = sh.tie_cnt[u][w];
        in_slot += cw;
        waves_before += w < wave ? cw : 0u;
      }
      const uint32_t k = kr[u];
      bool keep = k != 0 && (keep_all || k > thr);
      if (!keep && k != 0 && k == thr)
        keep = before + waves_before + (uint32_t)__popcll(tie_mask[u] & below) < ties_keep;
      if (keep) {
        const int beta = slots.block_of(u * kThreads + tid);
        atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
      }
      before += in_slot;
    }
  }
  emit_ids(p, unit, T, nb, bitmap, sh);
}

// Top-k + window + ascending ids for one unit, by the whole workgroup.
__device__ __forceinline__ void select_unit(const SelectParams& p, int unit, int T, const SlotMap& slots, int n,
                            TopkShared& sh, uint32_t* dyn) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int nb = slots.nb;
  const int words = (nb + 31) / 32;
  uint32_t* bitmap = dyn;                          // p.out_blocks_max bits
  uint32_t* sk = dyn + (p.out_blocks_max + 31) / 32;  // keys, when they fit
  const bool lds_keys = p.n_slots_max <= kLdsKeys;  // matches the launch's LDS size
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;  // published by the scoring
  for (int w = tid; w < words; w += kThreads) bitmap[w] = 0u;

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
      const uint32_t k = c < n && slots.block_of(c) >= 0 ? order_key(v[u]) : 0u;
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
    return slots.block_of(c) >= 0 ? order_key(published(&sc[c])) : 0u;
  };
  const uint32_t k_eff = min((uint32_t)max(p.top_k, 0), n_valid);
  const bool keep_none = k_eff == 0;
  const bool keep_all = !keep_none && k_eff == n_valid;

  // 2. the k-th largest key `thr` and how many keys equal to it are kept
  uint32_t thr = 0, ties_keep = 0;
  if (!keep_none && !keep_all && kmax == kmin) {
    thr = kmax;
    ties_keep = k_eff;
  } else if (!keep_none && !keep_all) {
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
      for (int c = tid; c < n; c += kThreads) {
        const uint32_t k = key_of(c);
        if (k == 0) continue;
        if (hi < 32 && (k >> hi) != (prefix >> hi)) continue;
        atomicAdd(&sh.hist[hist_slot((k >> shift) & (uint32_t)(nbins - 1))], 1u);
      }
      __syncthreads();
      take_digit(sh, nbins, shift, prefix, remaining);
    }
    thr = prefix;
    ties_keep = remaining;
  }

  // 3. mark kept blocks; thread t scans candidates [t*per, (t+1)*per) in order
  if (!keep_none) {
    const int per = (n + kThreads - 1) / kThreads;
    const int c0 = tid * per, c1 = min(c0 + per, n);
    uint32_t ties = 0;
    if (!keep_all)
      for (int c = c0; c < c1; ++c) ties += key_of(c) == thr ? 1u : 0u;
    uint32_t tot;
    uint32_t rank = block_excl_scan(ties, &tot, sh);
    for (int c = c0; c < c1; ++c) {
      const uint32_t k = key_of(c);
      if (k == 0) continue;
      bool keep = keep_all || k > thr;
      if (!keep && k == thr) keep = rank++ < ties_keep;
      if (keep) {
        const int beta = slots.block_of(c);
        atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
      }
    }
  }
  emit_ids(p, unit, T, nb, bitmap, sh);
}

// TS: storage type of a summary element (float for mean rows, TE for boxes)
// One scoring task: rows [chunk * kRowsPerWG, (chunk + 1) * kRowsPerWG) of
// the unit's candidate slots, by the whole workgroup. Every task of the unit
// (nchunks of them) arrives on the unit's counter; the last one to arrive
// runs the top-k and returns true (in every thread), having written the
// unit's ids and count with plain stores.
template <typename TE, int D, int KIND, int G>
__device__ __forceinline__ bool select_task(const SelectParams& p, int unit, int chunk, int nchunks,
                            TopkShared& sh, uint32_t* dyn) {
  using TS = typename std::conditional<KIND == HS_SUMMARY_MEAN, float, TE>::type;
  constexpr int EPS = 16 / sizeof(TS);                        // elements per 16-byte load
  constexpr int ROW = (KIND == HS_SUMMARY_MEAN ? 1 : 2) * D;  // elements per row
  constexpr int LPR = ROW / EPS;                              // lanes per row
  constexpr int RPW = kWave / LPR;                            // rows per wave instruction
  const KvView& kv = p.kv;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int T = clamp_len(kv, b);
  int nb = (T + p.block_size - 1) / p.block_size;
  nb = nb < p.out_blocks_max ? nb : p.out_blocks_max;
  const SlotMap slots = make_slots(p, unit, nb);
  int n_slots = p.gamma ? slots.gcnt * p.ratio : nb;
  n_slots = n_slots < p.n_slots_max ? n_slots : p.n_slots_max;
  const int c_begin = (chunk * kWaves + wave) * kRowsPerWave;

  static_assert(kRowsPerWG <= kThreads, "at most one staged score per thread");
  if (c_begin < n_slots) {  // wave-uniform
    const int li = lane % LPR, rg = lane / LPR;
    const int e0 = li * EPS;                                 // first element of the lane
    const int part = KIND == HS_SUMMARY_MEAN ? 0 : e0 / D;   // 0: min (or mean), 1: max
    const int dim0 = e0 % D;
    float coef[EPS];
#pragma unroll
    for (int k = 0; k < EPS; ++k) {
      float c = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float qv = load_elem<TE>(
            p.q, ((int64_t)b * kv.num_kv_heads * G + g * G + j) * D + dim0 + k);
        if (KIND == HS_SUMMARY_MEAN) c += qv;
        else c += part == 0 ? fminf(qv, 0.f) : fmaxf(qv, 0.f);
      }
      coef[k] = c;
    }
    const uint8_t* summ = reinterpret_cast<const uint8_t*>(p.summ) +
                          (int64_t)unit * p.max_blocks * ROW * sizeof(TS);
    const int c_end = min(c_begin + kRowsPerWave, n_slots);
    const int c_wg = chunk * kRowsPerWG;  // first slot of the workgroup
    for (int cb = c_begin; cb < c_end; cb += RPW * kUnroll) {
      uint4 r[kUnroll];
      int cs[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = cb + u * RPW + rg;
        const int beta = c < c_end ? slots.block_of(c) : -1;
        cs[u] = beta >= 0 ? c : -1;
        r[u] = beta >= 0 ? *reinterpret_cast<const uint4*>(
                               summ + (int64_t)beta * ROW * sizeof(TS) + li * 16)
                         : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float f[EPS];
        Vec16<TS>::unpack(r[u], f);
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < EPS; ++k) acc = fmaf(coef[k], f[k], acc);
        acc = group_sum<LPR>(acc);
        if (li == 0 && cs[u] >= 0) sh.stage[cs[u] - c_wg] = acc;
      }
    }
  }
  // publish the workgroup's scores with one coalesced store per thread
  __syncthreads();
  {
    const int c = chunk * kRowsPerWG + tid;
    if (tid < kRowsPerWG && c < n_slots)
      publish(&p.scores[(int64_t)unit * p.n_slots_max + c], sh.stage[tid]);
  }
  // every workgroup of the unit arrives; the last one selects
  if (!arrive_last(&p.counters[unit], nchunks, &sh.last)) return false;
  if (n_slots <= kThreads * kRegKeys)
    select_unit_regs<kRegKeys>(p, unit, T, slots, n_slots, sh, dyn);
  else
    select_unit(p, unit, T, slots, n_slots, sh, dyn);
  return true;
}

// Number of scoring tasks of a unit for a level with n_slots_max candidates.
__host__ __device__ inline int select_chunks(int n_slots_max) {
  return (n_slots_max + kRowsPerWG - 1) / kRowsPerWG;
}

}  // namespace
}  // namespace hs
