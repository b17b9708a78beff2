// summaries.hip - stage 1: per-block key summaries from the paged K cache.
//
// Mean-pooled keys ("SparDA" article, section 3.1; "8x256K ... porting
// HiSparse to QSA", section 2.2) and the per-dimension key min/max box of
// Quest ("SGLang hierarchical sparse attention", section 3.1.2), built in the
// representation phase of that page's section 2.2 and refreshed for the last,
// growing block while decoding.
//
// Mapping: one wave per block. A token row (head_dim elements) is read by
// LPT lanes with one 16-byte load each, so a wave instruction covers TPW
// consecutive tokens of the block; each lane reduces its token subset in
// registers, then the TPW token groups are combined across lanes. Reading K
// is the whole cost: the kernel streams each block's rows once, coalesced.
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kWavesPerWG = 4;
constexpr int kUnroll = 8;

template <typename TE, int D, int KIND>
__global__ __launch_bounds__(256) void k_build_summaries(SummParams p) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;   // lanes per token row
  constexpr int TPW = kWave / LPT;  // tokens per wave instruction
  const KvView& kv = p.kv;
  const int unit = blockIdx.y;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int S = p.block_size;
  const int beta = p.block_begin + blockIdx.x * kWavesPerWG + wave;
  const int T = clamp_len(kv, b);
  const int nb = (T + S - 1) / S;
  if (beta >= nb || beta >= p.max_blocks) return;
  const int tg = lane / LPT, li = lane % LPT;
  const int t0 = beta * S, t1 = min(t0 + S, T);

  float acc0[EPL], acc1[EPL];  // mean: sum in acc0; minmax: min in acc0, max in acc1
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    acc0[k] = KIND == HS_SUMMARY_MEAN ? 0.f : INFINITY;
    acc1[k] = -INFINITY;
  }
  for (int base = t0 + tg; base < t1; base += TPW * kUnroll) {
    uint4 r[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + u * TPW;
      const int64_t off = t < t1 ? row_offset(kv, b, g, t) : -1;
      ok[u] = off >= 0;
      r[u] = ok[u] ? *reinterpret_cast<const uint4*>(kv.k_pool + off + li * 16)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!ok[u]) continue;
      float f[EPL];
      Vec16<TE>::unpack(r[u], f);
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        if (KIND == HS_SUMMARY_MEAN) {
          acc0[k] += f[k];
        } else {
          acc0[k] = fminf(acc0[k], f[k]);
          acc1[k] = fmaxf(acc1[k], f[k]);
        }
      }
    }
  }
  // combine the TPW token groups (lanes LPT, 2 LPT, ... apart)
#pragma unroll
  for (int s = LPT; s < kWave; s *= 2) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float o0 = __shfl_xor(acc0[k], s);
      if (KIND == HS_SUMMARY_MEAN) {
        acc0[k] += o0;
      } else {
        const float o1 = __shfl_xor(acc1[k], s);
        acc0[k] = fminf(acc0[k], o0);
        acc1[k] = fmaxf(acc1[k], o1);
      }
    }
  }
  if (tg != 0) return;
  const int64_t row = (int64_t)unit * p.max_blocks + beta;
  if (KIND == HS_SUMMARY_MEAN) {
    const float n = (float)(t1 - t0);
    float* out = reinterpret_cast<float*>(p.out) + row * D + li * EPL;
#pragma unroll
    for (int k = 0; k < EPL; k += 4)
      *reinterpret_cast<float4*>(out + k) =
          make_float4(acc0[k] / n, acc0[k + 1] / n, acc0[k + 2] / n, acc0[k + 3] / n);
  } else {
    // min and max of stored values are stored values: write them back exactly
    uint4 lo, hi;
    if constexpr (EPL == 4) {
      lo = make_uint4(__float_as_uint(acc0[0]), __float_as_uint(acc0[1]),
                      __float_as_uint(acc0[2]), __float_as_uint(acc0[3]));
      hi = make_uint4(__float_as_uint(acc1[0]), __float_as_uint(acc1[1]),
                      __float_as_uint(acc1[2]), __float_as_uint(acc1[3]));
    } else {
      auto pack = [](float a, float c) {
        return (__float_as_uint(a) >> 16) | (__float_as_uint(c) & 0xFFFF0000u);
      };
      lo = make_uint4(pack(acc0[0], acc0[1]), pack(acc0[2], acc0[3]), pack(acc0[4], acc0[5]),
                      pack(acc0[6], acc0[7]));
      hi = make_uint4(pack(acc1[0], acc1[1]), pack(acc1[2], acc1[3]), pack(acc1[4], acc1[5]),
                      pack(acc1[6], acc1[7]));
    }
    uint8_t* out = reinterpret_cast<uint8_t*>(p.out) + row * 2 * D * (int64_t)sizeof(TE);
    *reinterpret_cast<uint4*>(out + li * 16) = lo;
    *reinterpret_cast<uint4*>(out + D * sizeof(TE) + li * 16) = hi;
  }
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
