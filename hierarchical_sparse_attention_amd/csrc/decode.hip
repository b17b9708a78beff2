// decode.hip - stage 3 as one launch: grid (splits, units), one split task
// per workgroup; the unit's last task merges. The device code and its
// sources are in decode_impl.h.
#include "decode_impl.h"

namespace hs {
namespace {

template <int D, int G>
__global__ __launch_bounds__(256) void k_decode_bf16(DecodeParams p) {
  __shared__ DecodeShared<D, G> ds;
  decode_task_bf16<D, G>(p, blockIdx.y, blockIdx.x, 0, ds);
}

template <int D, int G>
__global__ __launch_bounds__(256) void k_decode_f32(DecodeParams p) {
  __shared__ DecodeShared<D, G> ds;
  decode_task_f32<D, G, f32_unroll<G>()>(p, blockIdx.y, blockIdx.x, 0, ds);
}

template <int D>
hipError_t launch_bf16(const DecodeParams& p, dim3 grid, hipStream_t s) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_decode_bf16<D, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_decode_bf16<D, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_decode_bf16<D, 4>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((k_decode_bf16<D, 8>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const DecodeParams& p, dim3 grid, hipStream_t s) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_decode_f32<D, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_decode_f32<D, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_decode_f32<D, 4>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((k_decode_f32<D, 8>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

// A workgroup takes about 512 tokens (each of its 4 waves a quarter of the
// blocks), so that every wave pipelines several 32-token stages; long id
// lists get more blocks per split so that a unit has at most kMaxSplits.
int decode_blocks_per_split(int block_size, int max_selected) {
  int bps = block_size >= 128 ? 4 : 4 * ((128 + block_size - 1) / block_size);
  const int need = (max_selected + kMaxSplits - 1) / kMaxSplits;
  if (bps < need) bps = (need + 3) / 4 * 4;
  return bps;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.max_splits, p.kv.batch * p.kv.num_kv_heads);
  if (p.kv.elem_bytes == 2)
    return p.kv.head_dim == 64 ? launch_bf16<64>(p, grid, s) : launch_bf16<128>(p, grid, s);
  return p.kv.head_dim == 64 ? launch_f32<64>(p, grid, s) : launch_f32<128>(p, grid, s);
}

}  // namespace hs
