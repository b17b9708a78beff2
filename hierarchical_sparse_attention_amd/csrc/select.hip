// select.hip - stage 2: score every block against the query, keep a top-k
// (lowest block index wins ties) and add the window.
//
// Sources: "8x256K ... porting HiSparse to QSA" sections 2.2 (coarse level,
// fine level inside the kept coarse blocks, window level, merged), 3.2
// (selection moved to the GPU: block dot products then a top-k) and 5.1 (fp32
// scores compared at full precision); "SGLang hierarchical sparse attention"
// section 3.1.2 (Quest box bound); untitled HiSparse write-up section 3.3
// (window forced, then top-K in descending order).
//
// k_scores  - HBM stream of the summary table. Per unit the G query heads are
//             folded into per-dimension coefficients once (sum of q for mean
//             rows; sum of the negative / positive parts of q for the min /
//             max rows of a box, since max(q m, q M) = m min(q,0) + M max(q,0)),
//             so each summary element costs one FMA whatever G is. A row is
//             read by LPR lanes with 16-byte loads and reduced across them.
// k_topk    - one workgroup per unit. Exact radix select on order-preserving
//             uint32 keys of the fp32 scores: the leading bits shared by every
//             key are skipped, then 11-bit digits are resolved with an LDS
//             histogram until the k-th largest key is known. Keys above it are
//             kept; keys equal to it are kept in ascending candidate order
//             (candidate order is ascending block order), which realises the
//             lowest-index tie-break. Kept blocks and window blocks are set in
//             an LDS bitmap, which is written out as ascending ids.
#include <type_traits>

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kScoreRowsPerWave = 64;
constexpr int kScoreWaves = 4;
constexpr int kScoreUnroll = 8;

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

__device__ __forceinline__ SlotMap make_slots(const int32_t* gamma, const int32_t* gamma_cnt,
                                              int gamma_cap, int ratio, int unit, int nb) {
  SlotMap m;
  m.nb = nb;
  m.ratio = ratio;
  if (gamma) {
    int gc = gamma_cnt[unit];
    gc = gc < 0 ? 0 : (gc > gamma_cap ? gamma_cap : gc);
    m.gamma = gamma + (int64_t)unit * gamma_cap;
    m.gcnt = gc;
  } else {
    m.gamma = nullptr;
    m.gcnt = 0;
  }
  return m;
}

template <typename TE>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (sizeof(TE) == 4) return reinterpret_cast<const float*>(base)[i];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// TS: storage type of a summary element (float for mean rows, TE for boxes)
template <typename TE, int D, int KIND, int G>
__global__ __launch_bounds__(256) void k_scores(ScoreParams p) {
  using TS = typename std::conditional<KIND == HS_SUMMARY_MEAN, float, TE>::type;
  constexpr int EPS = 16 / sizeof(TS);                     // elements per 16-byte load
  constexpr int ROW = (KIND == HS_SUMMARY_MEAN ? 1 : 2) * D;  // elements per row
  constexpr int LPR = ROW / EPS;                           // lanes per row
  constexpr int RPW = kWave / LPR;                         // rows per wave instruction
  const KvView& kv = p.kv;
  const int unit = blockIdx.y;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int T = clamp_len(kv, b);
  const int nb = (T + p.block_size - 1) / p.block_size;
  const SlotMap slots = make_slots(p.gamma, p.gamma_cnt, p.gamma_cap, p.ratio, unit, nb);
  const int n_slots = p.gamma ? slots.gcnt * p.ratio : nb;
  const int c_begin = (blockIdx.x * kScoreWaves + wave) * kScoreRowsPerWave;
  if (c_begin >= n_slots) return;

  const int li = lane % LPR, rg = lane / LPR;
  const int e0 = li * EPS;                          // first element of this lane in a row
  const int part = KIND == HS_SUMMARY_MEAN ? 0 : e0 / D;  // 0: min (or mean), 1: max
  const int dim0 = e0 % D;
  float coef[EPS];
#pragma unroll
  for (int k = 0; k < EPS; ++k) {
    float c = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float qv = load_elem<TE>(p.q, ((int64_t)b * kv.num_kv_heads * G + g * G + j) * D +
                                              dim0 + k);
      if (KIND == HS_SUMMARY_MEAN) c += qv;
      else c += part == 0 ? fminf(qv, 0.f) : fmaxf(qv, 0.f);
    }
    coef[k] = c;
  }

  const uint8_t* summ = reinterpret_cast<const uint8_t*>(p.summ) +
                        (int64_t)unit * p.max_blocks * ROW * sizeof(TS);
  const int c_end = min(c_begin + kScoreRowsPerWave, n_slots);
  float* out = p.scores + (int64_t)unit * p.n_slots_max;
  for (int cb = c_begin; cb < c_end; cb += RPW * kScoreUnroll) {
    uint4 r[kScoreUnroll];
    int cs[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int c = cb + u * RPW + rg;
      const int beta = c < c_end ? slots.block_of(c) : -1;
      cs[u] = beta >= 0 ? c : -1;
      r[u] = beta >= 0 ? *reinterpret_cast<const uint4*>(summ + (int64_t)beta * ROW * sizeof(TS) +
                                                         li * 16)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float f[EPS];
      Vec16<TS>::unpack(r[u], f);
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < EPS; ++k) acc = fmaf(coef[k], f[k], acc);
      acc = group_sum<LPR>(acc);
      if (li == 0 && cs[u] >= 0) out[cs[u]] = acc;
    }
  }
}

// --------------------------------------------------------------------- top-k
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t wave_tot[kTopkWaves];
  uint32_t red_u[3][kTopkWaves];
  uint32_t bcast[4];
};

// Inclusive prefix sum over the wave (64 lanes).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int s = 1; s < kWave; s *= 2) {
    const uint32_t y = __shfl_up(x, s);
    if (lane >= s) x += y;
  }
  return x;
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t* total, TopkShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == kWave - 1) sh.wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t v = lane < kTopkWaves ? sh.wave_tot[lane] : 0u;
    const uint32_t vi = wave_incl_scan(v);
    if (lane < kTopkWaves) sh.wave_tot[lane] = vi - v;  // exclusive wave offsets
    if (lane == kTopkWaves - 1) sh.bcast[3] = vi;
  }
  __syncthreads();
  const uint32_t r = sh.wave_tot[wave] + inc - x;
  *total = sh.bcast[3];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t wave_sum_u(uint32_t x) {
#pragma unroll
  for (int s = 1; s < kWave; s *= 2) x += __shfl_xor(x, s);
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) {
#pragma unroll
  for (int s = 1; s < kWave; s *= 2) x = max(x, (uint32_t)__shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t x) {
#pragma unroll
  for (int s = 1; s < kWave; s *= 2) x = min(x, (uint32_t)__shfl_xor(x, s));
  return x;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(TopkParams p) {
  const int32_t out_blocks_max = p.out_blocks_max;
  __shared__ TopkShared sh;
  extern __shared__ uint32_t bitmap[];  // out_blocks_max bits
  const KvView& kv = p.kv;
  const int unit = blockIdx.x;
  const int b = unit / kv.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int T = clamp_len(kv, b);
  const int S = p.block_size;
  int nb = (T + S - 1) / S;
  nb = nb < out_blocks_max ? nb : out_blocks_max;
  const SlotMap slots = make_slots(p.gamma, p.gamma_cnt, p.gamma_cap, p.ratio, unit, nb);
  int n = p.gamma ? slots.gcnt * p.ratio : nb;
  n = n < p.n_slots_max ? n : p.n_slots_max;
  const float* sc = p.scores + (int64_t)unit * p.n_slots_max;
  const int words = (out_blocks_max + 31) / 32;
  for (int w = tid; w < words; w += kTopkThreads) bitmap[w] = 0u;

  auto key_of = [&](int c) -> uint32_t {  // 0 = not a candidate
    return slots.block_of(c) >= 0 ? order_key(sc[c]) : 0u;
  };

  // 1. number of candidates, largest and smallest key
  uint32_t cnt = 0, kmax = 0, kmin = 0xFFFFFFFFu;
  for (int c = tid; c < n; c += kTopkThreads) {
    const uint32_t k = key_of(c);
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
    sh.red_u[0][wave] = cnt;
    sh.red_u[1][wave] = kmax;
    sh.red_u[2][wave] = kmin;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0, mx = 0, mn = 0xFFFFFFFFu;
    for (int w = 0; w < kTopkWaves; ++w) {
      a += sh.red_u[0][w];
      mx = max(mx, sh.red_u[1][w]);
      mn = min(mn, sh.red_u[2][w]);
    }
    sh.bcast[0] = a;
    sh.bcast[1] = mx;
    sh.bcast[2] = mn;
  }
  __syncthreads();
  const uint32_t n_valid = sh.bcast[0];
  kmax = sh.bcast[1];
  kmin = sh.bcast[2];
  const uint32_t k_eff = min((uint32_t)max(p.top_k, 0), n_valid);

  // 2. the k-th largest key `thr` and how many keys equal to it are kept
  uint32_t thr = 0, ties_keep = 0;
  const bool keep_none = k_eff == 0;
  const bool keep_all = !keep_none && k_eff == n_valid;
  if (!keep_none && !keep_all && kmax == kmin) {  // all keys equal: lowest ids win
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
      const int hi = shift + db;  // bits at and above `hi` must equal prefix
      const uint32_t nbins = 1u << db;
      for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0u;
      __syncthreads();
      for (int c = tid; c < n; c += kTopkThreads) {
        const uint32_t k = key_of(c);
        if (k == 0) continue;
        if (hi < 32 && (k >> hi) != (prefix >> hi)) continue;
        atomicAdd(&sh.hist[(k >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      // suffix counts from the top bin down: thread t owns bins top-2t, top-2t-1.
      // Exactly one bin d has above(d) < remaining <= above(d) + hist[d].
      const int bA = (int)nbins - 1 - 2 * tid, bB = bA - 1;
      const uint32_t hA = bA >= 0 ? sh.hist[bA] : 0u, hB = bB >= 0 ? sh.hist[bB] : 0u;
      uint32_t tot;
      const uint32_t above = block_excl_scan(hA + hB, &tot, sh);
      if (bA >= 0 && above < remaining && above + hA >= remaining) {
        sh.bcast[0] = (uint32_t)bA;
        sh.bcast[1] = above;
      } else if (bB >= 0 && above + hA < remaining && above + hA + hB >= remaining) {
        sh.bcast[0] = (uint32_t)bB;
        sh.bcast[1] = above + hA;
      }
      __syncthreads();
      prefix |= sh.bcast[0] << shift;
      remaining -= sh.bcast[1];
      __syncthreads();
    }
    thr = prefix;
    ties_keep = remaining;
  }

  // 3. mark kept blocks in ascending candidate order (ties: lowest first)
  uint32_t run = 0;
  for (int c0 = 0; c0 < n; c0 += kTopkThreads) {
    const int c = c0 + tid;
    const uint32_t k = c < n ? key_of(c) : 0u;
    const bool tie = !keep_all && !keep_none && k != 0 && k == thr;
    uint32_t tot;
    const uint32_t rank = block_excl_scan(tie ? 1u : 0u, &tot, sh);
    bool keep;
    if (keep_none) keep = false;
    else if (keep_all) keep = k != 0;
    else keep = k != 0 && (k > thr || (tie && run + rank < ties_keep));
    if (keep) {
      const int beta = slots.block_of(c);
      atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
    }
    run += tot;
  }
  // 4. window: blocks holding any of the last W tokens
  if (p.window > 0) {
    const int64_t lo_tok = (int64_t)T - p.window;
    const int w0 = lo_tok <= 0 ? 0 : (int)(lo_tok / S);
    for (int beta = w0 + tid; beta < nb; beta += kTopkThreads)
      atomicOr(&bitmap[beta >> 5], 1u << (beta & 31));
  }
  __syncthreads();
  // 5. ascending ids
  int32_t* ids = p.out_ids + (int64_t)unit * p.out_cap;
  uint32_t base = 0;
  for (int w0 = 0; w0 < words; w0 += kTopkThreads) {
    const int w = w0 + tid;
    const uint32_t bits = w < words ? bitmap[w] : 0u;
    uint32_t tot;
    uint32_t pos = base + block_excl_scan(__popc(bits), &tot, sh);
    uint32_t m = bits;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)p.out_cap) ids[pos] = w * 32 + bit;
      ++pos;
    }
    base += tot;
  }
  if (tid == 0) p.out_cnt[unit] = (int32_t)min(base, (uint32_t)p.out_cap);
}

template <typename TE, int D, int KIND>
hipError_t launch_scores_g(const ScoreParams& p, dim3 grid, hipStream_t s) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_scores<TE, D, KIND, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_scores<TE, D, KIND, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_scores<TE, D, KIND, 4>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((k_scores<TE, D, KIND, 8>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

template <typename TE, int D>
hipError_t launch_scores_k(const ScoreParams& p, dim3 grid, hipStream_t s) {
  return p.kind == HS_SUMMARY_MEAN ? launch_scores_g<TE, D, HS_SUMMARY_MEAN>(p, grid, s)
                                   : launch_scores_g<TE, D, HS_SUMMARY_MINMAX>(p, grid, s);
}

}  // namespace

hipError_t launch_scores(const ScoreParams& p, hipStream_t s) {
  const int rows_per_wg = kScoreRowsPerWave * kScoreWaves;
  dim3 grid((p.n_slots_max + rows_per_wg - 1) / rows_per_wg, p.kv.batch * p.kv.num_kv_heads);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_scores_k<bf16_t, 64>(p, grid, s) : launch_scores_k<float, 64>(p, grid, s);
  return bf ? launch_scores_k<bf16_t, 128>(p, grid, s) : launch_scores_k<float, 128>(p, grid, s);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  const size_t lds = sizeof(uint32_t) * (size_t)((p.out_blocks_max + 31) / 32);
  hipLaunchKernelGGL(k_topk, dim3(p.kv.batch * p.kv.num_kv_heads), dim3(kTopkThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace hs
