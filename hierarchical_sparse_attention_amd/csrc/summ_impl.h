// summ_impl.h - device code of stage 1: the summary row of one block,
// computed by one wave from the paged K cache and stored; shared by the
// summary kernel and the scoring task that refreshes trailing blocks.
//
// Sources: mean-pooled keys ("SparDA" article, section 3.1; "8x256K ...
// porting HiSparse to QSA", section 2.2) and the per-dimension key min/max
// box of Quest ("SGLang hierarchical sparse attention", section 3.1.2).
//
// A token row (head_dim elements) is read by LPT lanes with one 16-byte load
// each, so a wave instruction covers TPW consecutive tokens of the block;
// each lane reduces its token subset in registers, then the TPW token groups
// are combined across lanes. Reading K is the whole cost: the block's rows
// are streamed once, coalesced.
#pragma once

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kSummUnroll = 8;

// Summary row of block beta (tokens [beta S, min(beta S + S, T))) of unit
// (b, g), by the calling wave, stored at row `row` of `out` (mean: float32
// [max_blocks][D] per unit; min/max: TE [max_blocks][2][D]).
template <typename TE, int D, int KIND>
__device__ __forceinline__ void summarize_block(const KvView& kv, void* out, int64_t row, int b,
                                                int g, int beta, int S, int T) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;      // lanes per token row
  constexpr int TPW = kWave / LPT;  // tokens per wave instruction
  const int lane = thread_id() & (kWave - 1);
  const int tg = lane / LPT, li = lane % LPT;
  const int t0 = beta * S, t1 = min(t0 + S, T);

  float acc0[EPL], acc1[EPL];  // mean: sum in acc0; minmax: min in acc0, max in acc1
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    acc0[k] = KIND == HS_SUMMARY_MEAN ? 0.f : INFINITY;
    acc1[k] = -INFINITY;
  }
  for (int base = t0 + tg; base < t1; base += TPW * kSummUnroll) {
    uint4 r[kSummUnroll];
    bool ok[kSummUnroll];
#pragma unroll
    for (int u = 0; u < kSummUnroll; ++u) {
      const int t = base + u * TPW;
      const int64_t off = t < t1 ? row_offset(kv, b, g, t) : -1;
      ok[u] = off >= 0;
      r[u] = ok[u] ? *reinterpret_cast<const uint4*>(kv.k_pool + off + li * 16)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kSummUnroll; ++u) {
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
  if (KIND == HS_SUMMARY_MEAN) {
    const float n = (float)(t1 - t0);
    float* o = reinterpret_cast<float*>(out) + row * D + li * EPL;
#pragma unroll
    for (int k = 0; k < EPL; k += 4)
      *reinterpret_cast<float4*>(o + k) =
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
    uint8_t* o = reinterpret_cast<uint8_t*>(out) + row * 2 * D * (int64_t)sizeof(TE);
    *reinterpret_cast<uint4*>(o + li * 16) = lo;
    *reinterpret_cast<uint4*>(o + D * sizeof(TE) + li * 16) = hi;
  }
}

}  // namespace
}  // namespace hs
