// summaries.hip - stage 1 as one launch: per-block key summaries from the
// paged K cache (grid: block groups x units), one wave per block, or one
// workgroup per block for blocks longer than a summation segment. The device
// code and its sources are in summ_impl.h; the representation phase builds
// every block, a decode step refreshes only the last, growing block.
#include "summ_impl.h"

namespace hs {
namespace {

constexpr int kWavesPerWG = 4;
constexpr int kBuildUnroll = 16;  // K loads in flight per lane (the values do not depend on it)

// Blocks of at most kSummSeg tokens: one wave per block, kWavesPerWG blocks
// per workgroup.
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
  summarize_block<TE, D, KIND, kBuildUnroll>(kv, p.out, (int64_t)unit * p.max_blocks + beta, b,
                                             g, beta, S, T);
}

// Longer blocks: one workgroup per block (summarize_block_wg).
template <typename TE, int D, int KIND>
__global__ __launch_bounds__(256) void k_build_long_summaries(SummParams p) {
  static_assert(kWavesPerWG == kSummWaves, "one block per workgroup of kSummWaves waves");
  constexpr int EPL = Vec16<TE>::EPL;
  __shared__ float seg[kSummWaves][2][D / EPL][EPL];  // per wave: [sum or min, max][lane][dim]
  const KvView& kv = p.kv;
  const int unit = blockIdx.y;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int S = p.block_size;
  const int beta = p.block_begin + blockIdx.x;
  const int T = clamp_len(kv, b);
  const int nb = (T + S - 1) / S;
  if (beta >= nb || beta >= p.max_blocks) return;  // uniform over the workgroup
  summarize_block_wg<TE, D, KIND, kBuildUnroll>(kv, p.out, (int64_t)unit * p.max_blocks + beta,
                                                b, g, beta, S, T, seg);
}

template <typename TE, int D>
hipError_t launch_td(const SummParams& p, dim3 grid, bool longb, hipStream_t s) {
  if (longb) {
    if (p.kind == HS_SUMMARY_MEAN)
      hipLaunchKernelGGL((k_build_long_summaries<TE, D, HS_SUMMARY_MEAN>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((k_build_long_summaries<TE, D, HS_SUMMARY_MINMAX>), grid, dim3(256), 0, s, p);
  } else if (p.kind == HS_SUMMARY_MEAN) {
    hipLaunchKernelGGL((k_build_summaries<TE, D, HS_SUMMARY_MEAN>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_build_summaries<TE, D, HS_SUMMARY_MINMAX>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_summaries(const SummParams& p, hipStream_t s) {
  const int S = p.block_size;
  const int nb_max = (p.kv.max_seq_len + S - 1) / S;
  const int n = (nb_max < p.max_blocks ? nb_max : p.max_blocks) - p.block_begin;
  if (n <= 0) return hipSuccess;
  const bool longb = S > kSummSeg;
  dim3 grid(longb ? n : (n + kWavesPerWG - 1) / kWavesPerWG, p.kv.batch * p.kv.num_kv_heads);
  const bool bf = p.kv.elem_bytes == 2;
  if (p.kv.head_dim == 64)
    return bf ? launch_td<bf16_t, 64>(p, grid, longb, s) : launch_td<float, 64>(p, grid, longb, s);
  return bf ? launch_td<bf16_t, 128>(p, grid, longb, s) : launch_td<float, 128>(p, grid, longb, s);
}

}  // namespace hs
