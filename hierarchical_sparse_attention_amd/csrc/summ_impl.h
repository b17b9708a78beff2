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

// 16 bytes at byte `col` of the rows of tokens t_u = first + u * step
// (u < N) of unit (b, g) in `pool`, for the tokens below t_end whose page is
// valid (ok[u]); the others read row 0 of page 0 instead (in bounds, ignored).
// All page-table loads are issued first and every row load after them, with
// no branch on loaded values, so the N round trips overlap.
template <int N>
__device__ __forceinline__ void load_rows(const KvView& kv, const uint8_t* pool, int b, int g,
                                          int first, int step, int t_end, int col,
                                          uint4 (&r)[N], bool (&ok)[N]) {
  int page[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int t = min(first + u * step, max(t_end - 1, 0));
    page[u] = kv.page_table[(int64_t)b * kv.max_pages + t / kv.page_size];
  }
  const int64_t row_bytes = (int64_t)kv.head_dim * kv.elem_bytes;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int t = first + u * step;
    ok[u] = t < t_end && (unsigned)page[u] < (unsigned)kv.num_phys_pages;
    const int64_t off = ok[u] ? (((int64_t)page[u] * kv.num_kv_heads + g) * kv.page_size +
                                 t % kv.page_size) * row_bytes
                              : 0;
    r[u] = *reinterpret_cast<const uint4*>(pool + off + col);
  }
}

// Summation order of a block's mean (every path that builds a summary row
// uses it, so the rows are bitwise equal whichever kernel built them): the
// block is cut into segments of kSummSeg tokens; inside a segment, lane group
// tg (of the TPW groups a 16-byte load instruction covers) adds the tokens
// tg, tg + TPW, ... in increasing order, and the groups are then combined
// across lanes; the segment sums are added in segment order. Min and max are
// exact in any order.
constexpr int kSummSeg = 128;

// Combined values of tokens [t_lo, t_hi) of unit (b, g) for this lane's
// dims (every lane ends with them): the sum (mean kinds) in acc0, or the
// min in acc0 and the max in acc1. U: K loads in flight per lane (any U
// gives the same values).
template <typename TE, int D, int KIND, int U>
__device__ __forceinline__ void summ_segment(const KvView& kv, int b, int g, int t_lo, int t_hi,
                                             float (&acc0)[Vec16<TE>::EPL],
                                             float (&acc1)[Vec16<TE>::EPL]) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;      // lanes per token row
  constexpr int TPW = kWave / LPT;  // tokens per wave instruction
  const int lane = thread_id() & (kWave - 1);
  const int tg = lane / LPT, li = lane % LPT;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    acc0[k] = KIND == HS_SUMMARY_MEAN ? 0.f : INFINITY;
    acc1[k] = -INFINITY;
  }
  for (int base = t_lo + tg; base < t_hi; base += TPW * U) {
    uint4 r[U];
    bool ok[U];
    load_rows<U>(kv, kv.k_pool, b, g, base, TPW, t_hi, li * 16, r, ok);
#pragma unroll
    for (int u = 0; u < U; ++u) {
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
}

// Folds a later segment's values into the running ones (segment order).
template <typename TE, int KIND>
__device__ __forceinline__ void summ_fold(float (&acc0)[Vec16<TE>::EPL],
                                          float (&acc1)[Vec16<TE>::EPL],
                                          const float (&s0)[Vec16<TE>::EPL],
                                          const float (&s1)[Vec16<TE>::EPL]) {
#pragma unroll
  for (int k = 0; k < Vec16<TE>::EPL; ++k) {
    if (KIND == HS_SUMMARY_MEAN) {
      acc0[k] += s0[k];
    } else {
      acc0[k] = fminf(acc0[k], s0[k]);
      acc1[k] = fmaxf(acc1[k], s1[k]);
    }
  }
}

// COHERENT: device-coherent stores (read by another workgroup of the launch)
template <typename TE, int D, int KIND, bool COHERENT = false>
__device__ __forceinline__ void summ_store(void* out, int64_t row,
                                           const float (&acc0)[Vec16<TE>::EPL],
                                           const float (&acc1)[Vec16<TE>::EPL], int n_tok);

// Summary row of block beta (tokens [beta S, min(beta S + S, T))) of unit
// (b, g), by the calling wave alone, segment after segment, stored at row
// `row` of `out` (mean: float32 [max_blocks][D] per unit; min/max: TE
// [max_blocks][2][D]).
template <typename TE, int D, int KIND, int U = kSummUnroll>
__device__ __forceinline__ void summarize_block(const KvView& kv, void* out, int64_t row, int b,
                                                int g, int beta, int S, int T) {
  constexpr int EPL = Vec16<TE>::EPL;
  const int t0 = beta * S, t1 = min(t0 + S, T);
  float acc0[EPL], acc1[EPL];
  if (KIND != HS_SUMMARY_MEAN) {  // min and max: one pass, any order
    summ_segment<TE, D, KIND, U>(kv, b, g, t0, t1, acc0, acc1);
  } else {
    summ_segment<TE, D, KIND, U>(kv, b, g, t0, min(t0 + kSummSeg, t1), acc0, acc1);
    for (int lo = t0 + kSummSeg; lo < t1; lo += kSummSeg) {
      float s0[EPL], s1[EPL];
      summ_segment<TE, D, KIND, U>(kv, b, g, lo, min(lo + kSummSeg, t1), s0, s1);
      summ_fold<TE, KIND>(acc0, acc1, s0, s1);
    }
  }
  summ_store<TE, D, KIND>(out, row, acc0, acc1, t1 - t0);
}

// Waves of a workgroup that builds one long block together.
constexpr int kSummWaves = 4;

// summarize_block for one block by a whole workgroup of kSummWaves waves
// (every thread calls it; blocks longer than a segment): in each round its
// waves reduce the next kSummWaves segments side by side and wave 0 folds
// them, in segment order, into the running values, so the row equals
// summarize_block's. seg: LDS scratch of the workgroup. COHERENT: the row is
// stored with device-coherent stores, for another workgroup of the launch.
template <typename TE, int D, int KIND, int U, bool COHERENT = false>
__device__ __forceinline__ void summarize_block_wg(
    const KvView& kv, void* out, int64_t row, int b, int g, int beta, int S, int T,
    float (*seg)[2][D / Vec16<TE>::EPL][Vec16<TE>::EPL]) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;
  const int wave = thread_id() / kWave, lane = thread_id() & (kWave - 1);
  const int t0 = beta * S, t1 = min(t0 + S, T);
  const int nseg = (t1 - t0 + kSummSeg - 1) / kSummSeg;
  float acc0[EPL], acc1[EPL];
  for (int r = 0; r < nseg; r += kSummWaves) {
    const int sg = r + wave;
    if (sg < nseg) {
      float s0[EPL], s1[EPL];
      const int lo = t0 + sg * kSummSeg;
      summ_segment<TE, D, KIND, U>(kv, b, g, lo, min(lo + kSummSeg, t1), s0, s1);
      if (lane < LPT) {  // token group 0 holds the segment's values
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          seg[wave][0][lane][k] = s0[k];
          seg[wave][1][lane][k] = s1[k];
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int li = lane % LPT;
      for (int w = 0; w < kSummWaves && r + w < nseg; ++w) {
        float s0[EPL], s1[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          s0[k] = seg[w][0][li][k];
          s1[k] = seg[w][1][li][k];
        }
        if (r + w == 0) {
#pragma unroll
          for (int k = 0; k < EPL; ++k) {
            acc0[k] = s0[k];
            acc1[k] = s1[k];
          }
        } else {
          summ_fold<TE, KIND>(acc0, acc1, s0, s1);
        }
      }
    }
    __syncthreads();
  }
  if (wave == 0) summ_store<TE, D, KIND, COHERENT>(out, row, acc0, acc1, t1 - t0);
}

// The same summary as summarize_block for a block of at most NL * TPW
// tokens, in two steps so that the loads can be issued early and used later:
// summ_load issues the block's K rows (NL 16-byte loads per lane, in the
// token order of summarize_block), summ_reduce folds them (every lane ends
// with the block's combined values for its dims, as in summarize_block before
// its store). Sums run in the same per-lane token order, so the results are
// bitwise those of summarize_block.
template <typename TE, int D, int NL>
__device__ __forceinline__ uint32_t summ_load(const KvView& kv, int b, int g, int beta, int S,
                                              int T, uint4 (&r)[NL]) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int TPW = kWave / LPT;
  const int lane = thread_id() & (kWave - 1);
  const int tg = lane / LPT, li = lane % LPT;
  const int t0 = beta * S, t1 = min(t0 + S, T);
  bool okb[NL];
  load_rows<NL>(kv, kv.k_pool, b, g, t0 + tg, TPW, t1, li * 16, r, okb);
  uint32_t ok = 0;
#pragma unroll
  for (int u = 0; u < NL; ++u) ok |= (okb[u] ? 1u : 0u) << u;
  return ok;
}

template <typename TE, int D, int KIND, int NL>
__device__ __forceinline__ void summ_reduce(const uint4 (&r)[NL], uint32_t ok,
                                            float (&acc0)[Vec16<TE>::EPL],
                                            float (&acc1)[Vec16<TE>::EPL]) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    acc0[k] = KIND == HS_SUMMARY_MEAN ? 0.f : INFINITY;
    acc1[k] = -INFINITY;
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    if (!((ok >> u) & 1u)) continue;
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
}

// Store of a reduced summary row (acc from summ_reduce; n valid tokens), as
// summarize_block stores it.
template <typename TE, int D, int KIND, bool COHERENT>
__device__ __forceinline__ void summ_store(void* out, int64_t row,
                                           const float (&acc0)[Vec16<TE>::EPL],
                                           const float (&acc1)[Vec16<TE>::EPL], int n_tok) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;
  const int lane = thread_id() & (kWave - 1);
  const int tg = lane / LPT, li = lane % LPT;
  if (tg != 0) return;
  if (KIND == HS_SUMMARY_MEAN) {
    const float n = (float)n_tok;
    float* o = reinterpret_cast<float*>(out) + row * D + li * EPL;
    if constexpr (COHERENT) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) publish(o + k, acc0[k] / n);
    } else {
#pragma unroll
      for (int k = 0; k < EPL; k += 4)
        *reinterpret_cast<float4*>(o + k) =
            make_float4(acc0[k] / n, acc0[k + 1] / n, acc0[k + 2] / n, acc0[k + 3] / n);
    }
  } else {
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
    if constexpr (COHERENT) {
      int32_t* w0 = reinterpret_cast<int32_t*>(o + li * 16);
      int32_t* w1 = reinterpret_cast<int32_t*>(o + D * sizeof(TE) + li * 16);
      const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, c[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        publish_i32(w0 + k, (int32_t)a[k]);
        publish_i32(w1 + k, (int32_t)c[k]);
      }
    } else {
      *reinterpret_cast<uint4*>(o + li * 16) = lo;
      *reinterpret_cast<uint4*>(o + D * sizeof(TE) + li * 16) = hi;
    }
  }
}

// The EPS stored values that the scoring layout puts in this lane (elements
// [li EPS, li EPS + EPS) of the row, li = lane % LPR), from a reduced
// summary: the values summ_store writes, read from registers. Min/max rows
// (and mean rows of float32 caches) hold a lane's elements in the lane
// itself; mean rows of bfloat16 caches take half of another lane's 8 dims.
template <typename TE, int D, int KIND, int EPS>
__device__ __forceinline__ void summ_row_elems(const float (&acc0)[Vec16<TE>::EPL],
                                               const float (&acc1)[Vec16<TE>::EPL], int n_tok,
                                               float (&f)[EPS]) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int ROW = (KIND == HS_SUMMARY_MEAN ? 1 : 2) * D;
  constexpr int LPR = ROW / EPS;
  const int lane = thread_id() & (kWave - 1);
  const int e0 = (lane % LPR) * EPS;
  const int part = e0 / D, d0 = e0 % D;
  const float n = (float)n_tok;
  if constexpr (EPS == EPL) {
#pragma unroll
    for (int k = 0; k < EPS; ++k)
      f[k] = KIND == HS_SUMMARY_MEAN ? acc0[k] / n : (part ? acc1[k] : acc0[k]);
  } else {
    static_assert(KIND == HS_SUMMARY_MEAN && EPS * 2 == EPL, "mean rows of a bf16 cache");
    const int src = d0 / EPL;  // a lane of token group 0 holding dims [src EPL, src EPL + EPL)
    const bool upper = (d0 % EPL) != 0;
#pragma unroll
    for (int k = 0; k < EPS; ++k) {
      const float lo = __shfl(acc0[k], src), hi = __shfl(acc0[k + EPS], src);
      f[k] = (upper ? hi : lo) / n;
    }
  }
}

}  // namespace
}  // namespace hs
