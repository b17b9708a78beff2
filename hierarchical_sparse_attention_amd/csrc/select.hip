// select.hip - stage 2 as one launch per selection level: grid (chunks,
// units), one scoring task per workgroup, the unit's last task selects.
// The device code and its sources are in select_impl.h.
#include "select_impl.h"

namespace hs {
namespace {

// dynamic LDS: [bitmap][keys of the general path][id list, out_cap + kWave]
template <typename TE, int D, int KIND, int G>
__global__ __launch_bounds__(kThreads) void k_select(SelectParams p, int list_off) {
  __shared__ TopkShared sh;
  extern __shared__ uint32_t dyn[];
  select_task<TE, D, KIND, G>(p, blockIdx.y, blockIdx.x, gridDim.x, sh, dyn,
                              reinterpret_cast<int32_t*>(dyn + list_off));
}

// One workgroup per unit: the pages of each selected block, in order, with the
// number of each page's tokens below the unit's length (0: no token, e.g. an
// absent entry, a page past T_b or an invalid page id).
__global__ __launch_bounds__(kThreads) void k_tok_pages(SelectParams p) {
  const int unit = blockIdx.x, b = unit / p.kv.num_kv_heads;
  const UnitGeom ug = unit_geom(p, unit);
  const int S = p.ratio, P = p.kv.page_size, ppb = p.tok_ppb;
  int2* out = p.tok_pages + (int64_t)unit * p.gamma_cap * ppb;
  for (int i = threadIdx.x; i < p.gamma_cap * ppb; i += kThreads) {
    const int gi = i / ppb, j = i - gi * ppb;
    int page = 0, lim = 0;
    const int gg = gi < ug.slots.gcnt ? ug.slots.gamma[gi] : -1;
    if (gg >= 0) {
      const int64_t t0 = (int64_t)gg * S + (int64_t)j * P;  // first token of the page
      if (t0 < ug.nb) {
        const int pg = p.kv.page_table[(int64_t)b * p.kv.max_pages + (int)(t0 / P)];
        if ((unsigned)pg < (unsigned)p.kv.num_phys_pages) {
          page = pg;
          lim = (int)min((int64_t)P, (int64_t)ug.nb - t0);
        }
      }
    }
    out[i] = make_int2(page, lim);
  }
}

template <typename TE, int D, int KIND>
hipError_t launch_g(const SelectParams& p, dim3 grid, size_t lds, int list_off, hipStream_t s) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_select<TE, D, KIND, 1>), grid, dim3(kThreads), lds, s, p, list_off); break;
    case 2: hipLaunchKernelGGL((k_select<TE, D, KIND, 2>), grid, dim3(kThreads), lds, s, p, list_off); break;
    case 4: hipLaunchKernelGGL((k_select<TE, D, KIND, 4>), grid, dim3(kThreads), lds, s, p, list_off); break;
    default: hipLaunchKernelGGL((k_select<TE, D, KIND, 8>), grid, dim3(kThreads), lds, s, p, list_off); break;
  }
  return hipGetLastError();
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

size_t select_launch_lds_bytes(int32_t out_blocks_max, int32_t n_slots_max, int32_t out_cap) {
  return select_lds_bytes(out_blocks_max, n_slots_max) + sizeof(uint32_t) * ((size_t)out_cap + kWave);
}

hipError_t launch_tok_pages(const SelectParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_tok_pages, dim3(p.kv.batch * p.kv.num_kv_heads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  const dim3 grid(select_chunks(p.n_slots_max),
                  p.kv.batch * p.kv.num_kv_heads);
  const int list_off = (int)(select_lds_bytes(p.out_blocks_max, p.n_slots_max) / sizeof(uint32_t));
  const size_t lds = sizeof(uint32_t) * ((size_t)list_off + p.out_cap + kWave);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_k<bf16_t, 64>(p, grid, lds, list_off, s)
              : launch_k<float, 64>(p, grid, lds, list_off, s);
  return bf ? launch_k<bf16_t, 128>(p, grid, lds, list_off, s)
            : launch_k<float, 128>(p, grid, lds, list_off, s);
}

}  // namespace hs
