// select.hip - stage 2 as one launch per selection level: grid (chunks,
// units), one scoring task per workgroup, the unit's last task selects.
// The device code and its sources are in select_impl.h.
#include "select_impl.h"

namespace hs {
namespace {

// dynamic LDS: [bitmap][keys of the general path][id list, out_cap + kWave]
// The token level asks for 3 waves per SIMD (at most 168 VGPRs), so that its
// (chunks x units) workgroups are resident together at the bench shapes.
template <typename TE, int D, int KIND, int G>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(KIND == kKindTokens ? 3 : 1))) void k_select(
    SelectParams p, int list_off) {
  __shared__ TopkShared sh;
  extern __shared__ uint32_t dyn[];
  select_task<TE, D, KIND, G>(p, blockIdx.y, blockIdx.x, gridDim.x, sh, dyn,
                              reinterpret_cast<int32_t*>(dyn + list_off));
}

static_assert(sizeof(TopkShared) + HS_TOKEN_LDS_BYTES <= (160u << 10),
              "a token-level workgroup fits the LDS of a gfx950 workgroup");

// Head of a two-level step (see HeadParams), two workgroups per unit. The
// builders (blocks [0, U)) rebuild the unit's growing coarse block(s), store
// them, count themselves on the unit's rebuilt_by word, then rebuild the
// growing fine block(s), which only the next launch reads. The selectors
// (blocks [U, 2U)) score the unit's coarse rows from the table as it is,
// wait for their builder's arrival, rescore the rebuilt rows with
// device-coherent loads, and select; the coarse candidates are one scoring
// chunk. Builders come first in the grid and never wait, so every
// selector's wait ends.
constexpr int kHeadUnroll = 16;  // K loads in flight per lane while rebuilding
template <typename TE, int D, int FKIND, int G>
__global__ __launch_bounds__(kThreads) void k_two_level_head(SelectParams p, HeadParams h,
                                                             int list_off) {
  constexpr int EPL = Vec16<TE>::EPL;
  static_assert(kThreads == kSummWaves * kWave, "one workgroup builds a long block");
  __shared__ union {
    TopkShared t;
    float seg[kSummWaves][2][D / EPL][EPL];
  } sh;
  extern __shared__ uint32_t dyn[];
  const KvView& kv = p.kv;
  const int U = kv.batch * kv.num_kv_heads;
  if (blockIdx.x >= U) {  // selector
    select_task<TE, D, HS_SUMMARY_MEAN, G>(p, blockIdx.x - U, 0, 1, sh.t, dyn,
                                           reinterpret_cast<int32_t*>(dyn + list_off));
    return;
  }
  const int unit = blockIdx.x;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int wave = thread_id() / kWave;
  const int T = clamp_len(kv, b);
  {  // coarse blocks: the whole workgroup each (uniform loop)
    const int S = p.block_size;
    const int nb = min((T + S - 1) / S, p.max_blocks);
    for (int beta = h.coarse_begin; beta < nb; ++beta)
      summarize_block_wg<TE, D, HS_SUMMARY_MEAN, kHeadUnroll, true>(  // read by the selector
          kv, const_cast<void*>(p.summ), (int64_t)unit * p.max_blocks + beta, b, g, beta, S, T,
          sh.seg);
    __builtin_amdgcn_s_waitcnt(0);  // the rebuilt rows are stored, device-coherently
    __syncthreads();
    // the selector waits exactly when its chunk holds a rebuilt row (same
    // unit_geom as the selector's)
    if (thread_id() == 0 && h.coarse_begin < unit_geom(p, unit).n)
      __hip_atomic_fetch_add(counter_of(p.rebuilt_by, unit), 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  {  // fine blocks: one wave each
    const int S = h.fine_block;
    const int nb = min((T + S - 1) / S, h.fine_max_blocks);
    for (int beta = h.fine_begin + wave; beta < nb; beta += kWaves)
      summarize_block<TE, D, FKIND, kHeadUnroll>(kv, h.fine, (int64_t)unit * h.fine_max_blocks + beta,
                                                 b, g, beta, S, T);
  }
}

template <typename TE, int D, int FKIND>
hipError_t launch_head_g(const SelectParams& p, const HeadParams& h, size_t lds, int list_off,
                         hipStream_t s) {
  const dim3 grid(2 * p.kv.batch * p.kv.num_kv_heads);  // builders, then selectors
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_two_level_head<TE, D, FKIND, 1>), grid, dim3(kThreads), lds, s, p, h, list_off); break;
    case 2: hipLaunchKernelGGL((k_two_level_head<TE, D, FKIND, 2>), grid, dim3(kThreads), lds, s, p, h, list_off); break;
    case 4: hipLaunchKernelGGL((k_two_level_head<TE, D, FKIND, 4>), grid, dim3(kThreads), lds, s, p, h, list_off); break;
    default: hipLaunchKernelGGL((k_two_level_head<TE, D, FKIND, 8>), grid, dim3(kThreads), lds, s, p, h, list_off); break;
  }
  return hipGetLastError();
}

template <typename TE, int D>
hipError_t launch_head_k(const SelectParams& p, const HeadParams& h, size_t lds, int list_off,
                         hipStream_t s) {
  return h.fine_kind == HS_SUMMARY_MEAN
             ? launch_head_g<TE, D, HS_SUMMARY_MEAN>(p, h, lds, list_off, s)
             : launch_head_g<TE, D, HS_SUMMARY_MINMAX>(p, h, lds, list_off, s);
}

template <typename TE, int D, int KIND, int G>
hipError_t launch_one(const SelectParams& p, dim3 grid, size_t lds, int list_off, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&k_select<TE, D, KIND, G>);
  if (lds > (64u << 10)) {  // above the default limit of dynamic LDS
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_select<TE, D, KIND, G>), grid, dim3(kThreads), lds, s, p, list_off);
  return hipGetLastError();
}

template <typename TE, int D, int KIND>
hipError_t launch_g(const SelectParams& p, dim3 grid, size_t lds, int list_off, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_one<TE, D, KIND, 1>(p, grid, lds, list_off, s);
    case 2: return launch_one<TE, D, KIND, 2>(p, grid, lds, list_off, s);
    case 4: return launch_one<TE, D, KIND, 4>(p, grid, lds, list_off, s);
    default: return launch_one<TE, D, KIND, 8>(p, grid, lds, list_off, s);
  }
}

template <typename TE, int D>
hipError_t launch_k(const SelectParams& p, dim3 grid, size_t lds, int list_off, hipStream_t s) {
  if (p.kind == kKindTokens) return launch_g<TE, D, kKindTokens>(p, grid, lds, list_off, s);
  return p.kind == HS_SUMMARY_MEAN ? launch_g<TE, D, HS_SUMMARY_MEAN>(p, grid, lds, list_off, s)
                                   : launch_g<TE, D, HS_SUMMARY_MINMAX>(p, grid, lds, list_off, s);
}

}  // namespace

size_t select_lds_bytes(int32_t out_blocks_max, int32_t n_slots_max) {
  const size_t words = (size_t)(out_blocks_max + 31) / 32;
  const bool general = n_slots_max > kThreads * kRegKeys;
  const size_t keys = general && n_slots_max <= kLdsKeys ? (size_t)n_slots_max : 0;
  return sizeof(uint32_t) * (words + keys);
}

bool tokens_in_registers(int32_t kind, int32_t n_slots_max, int32_t gamma_cap) {
  return kind == kKindTokens && n_slots_max <= kThreads * kTokKeys && gamma_cap <= kGammaLds;
}

size_t select_launch_lds_bytes(int32_t out_blocks_max, int32_t n_slots_max, int32_t out_cap) {
  return select_lds_bytes(out_blocks_max, n_slots_max) + sizeof(uint32_t) * ((size_t)out_cap + kWave);
}

bool two_level_head_fits(const SelectParams& coarse, int32_t fine_block, int32_t coarse_kind) {
  return coarse_kind == HS_SUMMARY_MEAN && fine_block <= kSummSeg &&
         select_chunks(coarse.n_slots_max) == 1 &&
         select_launch_lds_bytes(coarse.out_blocks_max, coarse.n_slots_max, coarse.out_cap) <=
             (48u << 10);
}

hipError_t launch_two_level_head(const SelectParams& coarse, const HeadParams& h, hipStream_t s) {
  // the selectors rescore the rows their builders rebuild: the rebuilt-row
  // arrivals take the second word of each unit's coarse counter line
  SelectParams p = coarse;
  p.refresh_begin = h.coarse_begin;
  p.rebuilt_by = coarse.counters + 1;
  p.status = h.status;
  const hipError_t e = wait_bound(&p.wait_ticks);
  if (e != hipSuccess) return e;
  const int list_off = (int)(select_lds_bytes(p.out_blocks_max, p.n_slots_max) / sizeof(uint32_t));
  const size_t lds = sizeof(uint32_t) * ((size_t)list_off + p.out_cap + kWave);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_head_k<bf16_t, 64>(p, h, lds, list_off, s)
              : launch_head_k<float, 64>(p, h, lds, list_off, s);
  return bf ? launch_head_k<bf16_t, 128>(p, h, lds, list_off, s)
            : launch_head_k<float, 128>(p, h, lds, list_off, s);
}

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  const dim3 grid(select_chunks(p.n_slots_max),
                  p.kv.batch * p.kv.num_kv_heads);
  const int list_off = (int)(select_lds_bytes(p.out_blocks_max, p.n_slots_max) / sizeof(uint32_t));
  // the token level's register path (topk_tokens) uses static LDS only
  const size_t lds = tokens_in_registers(p.kind, p.n_slots_max, p.gamma_cap)
                         ? 0
                         : sizeof(uint32_t) * ((size_t)list_off + p.out_cap + kWave);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_k<bf16_t, 64>(p, grid, lds, list_off, s)
              : launch_k<float, 64>(p, grid, lds, list_off, s);
  return bf ? launch_k<bf16_t, 128>(p, grid, lds, list_off, s)
            : launch_k<float, 128>(p, grid, lds, list_off, s);
}

}  // namespace hs
