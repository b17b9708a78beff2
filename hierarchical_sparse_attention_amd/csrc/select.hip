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
