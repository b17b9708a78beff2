// summaries.hip - stage 1 as one launch: per-block key summaries from the
// paged K cache, one wave per block (grid: block groups x units). The device
// code and its sources are in summ_impl.h; the representation phase builds
// every block, a decode step refreshes only the last, growing block.
#include "summ_impl.h"

namespace hs {
namespace {

constexpr int kWavesPerWG = 4;

template <typename TE, int D, int KIND>
__global__ __launch_bounds__(256) void k_build_summaries(SummParams p) {
  const KvView& kv = p.kv;
  const int unit = blockIdx.y;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int wave = threadIdx.x / kWave;
  const int S = p.block_size;
  const int beta = p.block_begin + blockIdx.x * kWavesPerWG + wave;
  const int T = clamp_len(kv, b);
  const int nb = (T + S - 1) / S;
  if (beta >= nb || beta >= p.max_blocks) return;
  summarize_block<TE, D, KIND>(kv, p.out, (int64_t)unit * p.max_blocks + beta, b, g, beta, S, T);
}

template <typename TE, int D>
hipError_t launch_td(const SummParams& p, dim3 grid, hipStream_t s) {
  if (p.kind == HS_SUMMARY_MEAN)
    hipLaunchKernelGGL((k_build_summaries<TE, D, HS_SUMMARY_MEAN>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_build_summaries<TE, D, HS_SUMMARY_MINMAX>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_summaries(const SummParams& p, hipStream_t s) {
  const int S = p.block_size;
  const int nb_max = (p.kv.max_seq_len + S - 1) / S;
  const int n = (nb_max < p.max_blocks ? nb_max : p.max_blocks) - p.block_begin;
  if (n <= 0) return hipSuccess;
  dim3 grid((n + kWavesPerWG - 1) / kWavesPerWG, p.kv.batch * p.kv.num_kv_heads);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_td<bf16_t, 64>(p, grid, s) : launch_td<float, 64>(p, grid, s);
  return bf ? launch_td<bf16_t, 128>(p, grid, s) : launch_td<float, 128>(p, grid, s);
}

}  // namespace hs
