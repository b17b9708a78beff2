// decode.hip - stage 3: exact softmax attention over the selected blocks,
// read in place from the paged KV cache.
//
// Sources: "8x256K ... porting HiSparse to QSA" section 3.3 (the attention
// loop walks a compact list of selected blocks instead of all blocks, with an
// online softmax) and section 2.3 (no gather of the selected KV into a
// compact copy); "SparDA" article section 3.3 (only the selected pages are
// read) and section 3.4 (one block list shared by every layer).
//
// k_decode_split - grid (splits, units). A workgroup owns a run of
//   blocks_per_split consecutive entries of a unit's id list (about 256
//   tokens) and computes, for the unit's G query heads, an fp32 online-softmax
//   partial (m, l, o) over them. Each wave takes every fourth entry. A token
//   row is read by LPT lanes with one 16-byte load each, so one wave
//   instruction covers TPW tokens; K and V loads for UNR such instructions
//   are issued before any use. The q.k dot is reduced across the LPT lanes
//   with DPP, which leaves the logit in every lane of the token's lane group:
//   each lane then accumulates p * v for its own head_dim slice without any
//   broadcast. Token groups, then waves, are merged at the end (LSE rule).
// k_decode_merge - one workgroup per (b, query head): log-sum-exp merge of
//   the unit's split partials into the fp32 output.
// Logits are kept in base 2: q is pre-multiplied by scale * log2(e), so
// exp(l - m) = exp2(l2 - m2) exactly in real arithmetic.
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kDecWaves = 4;

template <typename TE, int D, int G, int UNR>
__global__ __launch_bounds__(256) void k_decode_split(DecodeParams p) {
  constexpr int EPL = Vec16<TE>::EPL;
  constexpr int LPT = D / EPL;        // lanes per token row
  constexpr int TPW = kWave / LPT;    // tokens per wave instruction
  const KvView& kv = p.kv;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int T = clamp_len(kv, b);
  const int S = p.block_size;
  const int nb = (T + S - 1) / S;
  int cnt = p.counts[unit];
  cnt = cnt < 0 ? 0 : (cnt > p.max_selected ? p.max_selected : cnt);
  const int e0 = split * p.blocks_per_split;
  if (e0 >= cnt) return;  // no partial: the merge reads only splits below ceil(cnt / bps)
  const int e1 = min(e0 + p.blocks_per_split, cnt);

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int tg = lane / LPT, li = lane % LPT;
  const int Hq = kv.num_kv_heads * G;

  float qv[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) +
                        ((int64_t)b * Hq + g * G + j) * D * (int64_t)sizeof(TE) + li * 16;
    Vec16<TE>::unpack(*reinterpret_cast<const uint4*>(qp), qv[j]);
#pragma unroll
    for (int k = 0; k < EPL; ++k) qv[j][k] *= p.scale_log2;
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[j][k] = 0.f;
  }

  const int32_t* ids = p.ids + (int64_t)unit * p.max_selected;
  for (int e = e0 + wave; e < e1; e += kDecWaves) {
    const int beta = ids[e];
    if ((unsigned)beta >= (unsigned)nb) continue;  // wave-uniform
    const int tb = beta * S, te = min(tb + S, T);
    for (int t0 = tb; t0 < te; t0 += TPW * UNR) {  // wave-uniform trip count
      uint4 kr[UNR], vr[UNR];
      bool ok[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int t = t0 + u * TPW + tg;
        const int64_t off = t < te ? row_offset(kv, b, g, t) : -1;
        ok[u] = off >= 0;
        kr[u] = ok[u] ? *reinterpret_cast<const uint4*>(kv.k_pool + off + li * 16)
                      : make_uint4(0, 0, 0, 0);
        vr[u] = ok[u] ? *reinterpret_cast<const uint4*>(kv.v_pool + off + li * 16)
                      : make_uint4(0, 0, 0, 0);
      }
      float x[UNR][G];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float kf[EPL];
        Vec16<TE>::unpack(kr[u], kf);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float a = 0.f;
#pragma unroll
          for (int k = 0; k < EPL; ++k) a = fmaf(qv[j][k], kf[k], a);
          a = group_sum<LPT>(a);
          x[u][j] = ok[u] ? a : -INFINITY;
        }
      }
      float pr[UNR][G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float mx = x[0][j];
#pragma unroll
        for (int u = 1; u < UNR; ++u) mx = fmaxf(mx, x[u][j]);
        const float mn = fmaxf(m[j], mx);
        // mn == -inf: nothing valid in this lane group yet; keep the state
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float alpha = exp2f(m[j] - ms);  // m = -inf -> 0
        m[j] = mn;
        l[j] *= alpha;
#pragma unroll
        for (int k = 0; k < EPL; ++k) o[j][k] *= alpha;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          pr[u][j] = exp2f(x[u][j] - ms);  // x = -inf -> 0
          l[j] += pr[u][j];
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float vf[EPL];
        Vec16<TE>::unpack(vr[u], vf);
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int k = 0; k < EPL; ++k) o[j][k] = fmaf(pr[u][j], vf[k], o[j][k]);
      }
    }
  }

  // merge the TPW token groups of the wave (lanes LPT, 2 LPT, ... apart)
#pragma unroll
  for (int s = LPT; s < kWave; s *= 2) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float m2 = __shfl_xor(m[j], s);
      const float l2 = __shfl_xor(l[j], s);
      const float mn = fmaxf(m[j], m2);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float a1 = exp2f(m[j] - ms), a2 = exp2f(m2 - ms);
      m[j] = mn;
      l[j] = l[j] * a1 + l2 * a2;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        const float o2 = __shfl_xor(o[j][k], s);
        o[j][k] = o[j][k] * a1 + o2 * a2;
      }
    }
  }

  // merge the waves through LDS and write this split's partial
  __shared__ float sh_o[kDecWaves][G][D];
  __shared__ float sh_m[kDecWaves][G], sh_l[kDecWaves][G];
  if (tg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) sh_o[wave][j][li * EPL + k] = o[j][k];
      if (li == 0) {
        sh_m[wave][j] = m[j];
        sh_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();
  const int64_t ps = (int64_t)unit * p.max_splits + split;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int j = idx / D, dd = idx % D;
    float mn = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mn = fmaxf(mn, sh_m[w][j]);
    const float ms = mn == -INFINITY ? 0.f : mn;
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float a = exp2f(sh_m[w][j] - ms);
      acc += sh_o[w][j][dd] * a;
      lsum += sh_l[w][j] * a;
    }
    p.part_o[(ps * G + j) * D + dd] = acc;
    if (dd == 0) {
      p.part_ml[(ps * G + j) * 2 + 0] = mn;
      p.part_ml[(ps * G + j) * 2 + 1] = lsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(128) void k_decode_merge(DecodeParams p) {
  const KvView& kv = p.kv;
  const int Hq = kv.num_kv_heads * p.G;
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int g = h / p.G, j = h % p.G;
  const int unit = b * kv.num_kv_heads + g;
  int cnt = p.counts[unit];
  cnt = cnt < 0 ? 0 : (cnt > p.max_selected ? p.max_selected : cnt);
  const int ns = (cnt + p.blocks_per_split - 1) / p.blocks_per_split;
  const int64_t p0 = (int64_t)unit * p.max_splits;
  float mn = -INFINITY;
  for (int s = 0; s < ns; ++s) mn = fmaxf(mn, p.part_ml[((p0 + s) * p.G + j) * 2]);
  const float ms = mn == -INFINITY ? 0.f : mn;
  for (int dd = threadIdx.x; dd < D; dd += blockDim.x) {
    float acc = 0.f, lsum = 0.f;
    for (int s = 0; s < ns; ++s) {
      const int64_t r = (p0 + s) * p.G + j;
      const float a = exp2f(p.part_ml[r * 2] - ms);
      acc += p.part_o[r * D + dd] * a;
      lsum += p.part_ml[r * 2 + 1] * a;
    }
    p.out[((int64_t)b * Hq + h) * D + dd] = lsum > 0.f ? acc / lsum : 0.f;
  }
}

template <typename TE, int D>
hipError_t launch_split(const DecodeParams& p, dim3 grid, hipStream_t s) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((k_decode_split<TE, D, 1, 8>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_decode_split<TE, D, 2, 8>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_decode_split<TE, D, 4, 8>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((k_decode_split<TE, D, 8, 4>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

int decode_blocks_per_split(int block_size) {
  const int bps = 256 / block_size;
  return bps < 1 ? 1 : bps;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  const int units = p.kv.batch * p.kv.num_kv_heads;
  dim3 grid(p.max_splits, units);
  const bool bf = p.kv.elem_bytes == 2;
  hipError_t e;
  if (p.kv.head_dim == 64)
    e = bf ? launch_split<bf16_t, 64>(p, grid, s) : launch_split<float, 64>(p, grid, s);
  else
    e = bf ? launch_split<bf16_t, 128>(p, grid, s) : launch_split<float, 128>(p, grid, s);
  if (e != hipSuccess) return e;
  const dim3 mgrid(p.kv.batch * p.kv.num_kv_heads * p.G);
  if (p.kv.head_dim == 64)
    hipLaunchKernelGGL(k_decode_merge<64>, mgrid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(k_decode_merge<128>, mgrid, dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs
