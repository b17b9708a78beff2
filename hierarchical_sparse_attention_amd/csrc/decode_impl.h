// decode_impl.h - device code of stage 3, exact softmax attention over the
// selected blocks read in place from the paged KV cache; shared by the decode
// kernel and the fused select-and-decode kernel.
//
// Sources: "8x256K ... porting HiSparse to QSA" section 3.3 (the attention
// loop walks a compact list of selected blocks instead of all blocks, with an
// online softmax) and section 2.3 (no gather of the selected KV into a
// compact copy); "SparDA" article section 3.3 (only the selected pages are
// read) and section 3.4 (one block list shared by every layer).
//
// Work split: a unit's id list is cut into n_splits equal runs of entries
// (by the unit's actual count); one workgroup task per (unit, split). The 4
// waves of a task take every fourth entry of the run and keep an fp32
// online-softmax state (m, l, o) for the unit's G query heads. The task
// combines its waves in LDS and publishes one partial; the last task of the
// unit to arrive (arrival counter in the workspace) merges the n_splits
// partials into the output with the log-sum-exp rule, so one launch does the
// whole stage.
//
// bf16 caches: q.k on the matrix cores. For a 16-token tile
// v_mfma_f32_16x16x32_bf16 takes the unit's query heads as rows of A (head j
// in row 4 (j % 4) + j / 4, so every 16-lane group of the result holds one
// head's 16 logits) and the K tile as B: each lane's 16-byte load of
// 8 consecutive dims of one token is exactly its B operand, so K goes from
// HBM to the MFMA without any shuffle. Softmax statistics are per head and
// wave-uniform; p and the rescale factor go through a small per-wave LDS
// slice to the p.v accumulation, which runs on the VALU in fp32 with V read
// as 16-byte rows (lane: 8 dims of one token).
// float32 caches: all on the VALU; the q.k dot is reduced across the lanes of
// a token row with DPP.
// Logits are kept in base 2: the logit scale is multiplied by log2(e), so
// exp(l - m) = exp2(l2 - m2) in real arithmetic.
#pragma once

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int D, int G>
struct SplitShared {
  float o[kDecWaves][G][D];
  float m[kDecWaves][G];
  float l[kDecWaves][G];
  int last;
};

// Entries [e0, e1) of a list of cnt entries owned by split `split` of ns:
// consecutive runs whose lengths differ by at most one.
__device__ __forceinline__ void split_range(int cnt, int ns, int split, int& e0, int& e1) {
  e0 = (int)((int64_t)cnt * split / ns);
  e1 = (int)((int64_t)cnt * (split + 1) / ns);
}

// Log-sum-exp merge of the unit's n_splits partials into `out`, by the unit's
// last-arriving task. Thread t owns output elements t + 256 e of the unit's
// G x D block; the partials of SB splits are loaded together (one round trip
// to the device-coherent level per batch), then folded in split order.
template <int D, int G>
__device__ __forceinline__ void merge_splits(const DecodeParams& p, int unit) {
  constexpr int E = G * D;
  constexpr int EPT = (E + kDecThreads - 1) / kDecThreads;
  constexpr int SB = 16 / EPT;
  const int tid = thread_id();
  const int ns = p.n_splits;
  const int64_t p0 = (int64_t)unit * ns;
  float m[EPT], l[EPT], o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.f;
    o[e] = 0.f;
  }
  for (int s0 = 0; s0 < ns; s0 += SB) {
    float ov[SB][EPT], mv[SB][EPT], lv[SB][EPT];
#pragma unroll
    for (int bt = 0; bt < SB; ++bt) {
      const int64_t s = p0 + min(s0 + bt, ns - 1);  // unconditional (clamped) loads overlap
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int idx = min(tid + kDecThreads * e, E - 1), j = idx / D;
        ov[bt][e] = published(&p.part_o[s * E + idx]);
        mv[bt][e] = published(&p.part_ml[(s * G + j) * 2]);
        lv[bt][e] = published(&p.part_ml[(s * G + j) * 2 + 1]);
      }
    }
#pragma unroll
    for (int bt = 0; bt < SB; ++bt) {
      if (s0 + bt >= ns) break;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float mn = fmaxf(m[e], mv[bt][e]);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float a = exp2f(m[e] - ms), c = exp2f(mv[bt][e] - ms);
        l[e] = l[e] * a + lv[bt][e] * c;
        o[e] = o[e] * a + ov[bt][e] * c;
        m[e] = mn;
      }
    }
  }
  const int Hq = p.kv.num_kv_heads * G;
  const int b = unit / p.kv.num_kv_heads, g = unit % p.kv.num_kv_heads;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int idx = tid + kDecThreads * e;
    if (idx < E) p.out[((int64_t)b * Hq + g * G) * D + idx] = l[e] > 0.f ? o[e] / l[e] : 0.f;
  }
}

// Combine the waves' states (in sh) into the task's partial, publish it and
// arrive on the unit's counter; the last of the n_splits tasks to arrive
// merges (and, in the fused launch, takes the unit's scoring arrivals off its
// scoring counter, which every task of the unit has read by then).
template <int D, int G>
__device__ __forceinline__ void finish_split(const DecodeParams& p, SplitShared<D, G>& sh, int unit,
                                             int split) {
  const int tid = thread_id();
  __syncthreads();
  const int64_t ps = (int64_t)unit * p.n_splits + split;
  for (int idx = tid; idx < G * D; idx += kDecThreads) {
    const int j = idx / D, dd = idx % D;
    float mn = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mn = fmaxf(mn, sh.m[w][j]);
    const float ms = mn == -INFINITY ? 0.f : mn;
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float a = exp2f(sh.m[w][j] - ms);
      acc += sh.o[w][j][dd] * a;
      lsum += sh.l[w][j] * a;
    }
    publish(&p.part_o[ps * G * D + idx], acc);
    if (dd == 0) {
      publish(&p.part_ml[(ps * G + j) * 2 + 0], mn);
      publish(&p.part_ml[(ps * G + j) * 2 + 1], lsum);
    }
  }
  if (!arrive_last(counter_of(p.counters, unit), p.n_splits, &sh.last)) return;
  // the scoring arrivals this call counted are taken off again (not stored as
  // zero), so the counter is zero for the next call even if a wait expired
  // before the last scoring task arrived
  if (p.score_counters != nullptr && tid == 0)
    __hip_atomic_fetch_add(counter_of(p.score_counters, unit), -p.score_chunks, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  merge_splits<D, G>(p, unit);
}

// --------------------------------------------------------------- bf16 path
// One 32-token stage of K and V as loaded (two 16-token MFMA tiles of K in
// B-operand layout, V as 16-byte rows).
template <int D>
struct StageRegs {
  uint4 k[2][D / 32];
  uint4 v[32 / (kWave / (D / 8))];
  uint32_t ok;  // token list mode: bit tau set if this lane's token 16 tau + r16 is valid
};

constexpr int kStagesPerChunk = kWave;  // stage-table entries filled per pass

// LDS of one split task (both paths; the float32 path uses `sh` only).
template <int D, int G>
struct DecodeShared {
  SplitShared<D, G> sh;
  float sp[kDecWaves][32][G];
  float salpha[kDecWaves][G];
  int64_t st_base[kDecWaves][kStagesPerChunk];  // see the stage table below
  int st_len[kDecWaves][kStagesPerChunk];
};

// Attention of the unit's query heads over the blocks ids[e0 .. e1) (a list
// in LDS or global memory) of a bf16 cache; leaves each wave's state in
// ds.sh for finish_split. TOK: the list is of single tokens (block size 1),
// given as the byte offsets of their rows, rows[e0 .. e1), resolved by the
// caller; a masked token's entry is ~r, r the offset of a finite row its
// lane reads instead.
template <int D, int G, bool TOK>
__device__ __forceinline__ void attend_bf16(const DecodeParams& p, int unit, const int32_t* ids,
                                            int e0, int e1, DecodeShared<D, G>& ds,
                                            const int64_t* rows) {
  constexpr int KC = D / 32;       // MFMA k-chunks per token row
  constexpr int VL = D / 8;        // lanes per V row (16 bytes each)
  constexpr int TPV = kWave / VL;  // tokens per V load instruction
  constexpr int NV = 32 / TPV;     // V loads per 32-token stage
  constexpr int GR = (G + 3) / 4;  // MFMA result registers that carry heads
  constexpr int EB = 2;            // bytes per element
  SplitShared<D, G>& sh = ds.sh;
  auto& sp = ds.sp;
  auto& salpha = ds.salpha;
  auto& st_base = ds.st_base;
  auto& st_len = ds.st_len;

  const KvView& kv = p.kv;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int T = clamp_len(kv, b);
  const int S = p.block_size;
  const int nb = (T + S - 1) / S;
  const int tid = thread_id();
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r16 = lane & 15, grp = lane >> 4;
  const int vt = lane / VL, vd = (lane % VL) * 8;
  const int Hq = kv.num_kv_heads * G;
  const float scale = p.scale_log2;
  // a 32-token stage stays inside one page when the page and block sizes are
  // multiples of 32: then one page lookup serves the whole stage
  const bool whole_page = (kv.page_size % 32 == 0) && (S % 32 == 0);
  // block size 1 (a token list, e.g. from the token-level second stage): a
  // stage is up to 32 consecutive list entries, each lane reads its own
  // token's row offset from `rows`; masked tokens (outside [0, T) or on an
  // absent page) read the finite row their entry names
  constexpr bool tok_list = TOK;
  const int64_t row_bytes = (int64_t)D * EB;

  // A operands: query head j in row 4 (j % 4) + j / 4 (zero rows elsewhere)
  bf16x8_t aq[KC];
  {
    const int j = 4 * (r16 & 3) + (r16 >> 2);
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) +
                          ((int64_t)b * Hq + g * G + (j < G ? j : 0)) * row_bytes;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 r = j < G ? *reinterpret_cast<const uint4*>(qrow + (32 * c + 8 * grp) * EB)
                      : make_uint4(0, 0, 0, 0);
      aq[c] = __builtin_bit_cast(bf16x8_t, r);
    }
  }
  float m_run[GR], l_run[GR], o[G][8];
#pragma unroll
  for (int i = 0; i < GR; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) o[j][k] = 0.f;

  // Issue the loads of stage `st` of the table. Lanes of masked tokens load a
  // valid row of the same stage instead (their logits are -inf, so their p is
  // 0 and the finite V row adds nothing); an empty stage loads nothing.
  // (a token list names its masked tokens' stand-in rows itself)
  const int64_t row0 = !TOK && T > 0 ? max(row_offset(kv, b, g, 0), (int64_t)0) : 0;
  // byte offset of the row of list entry `e` (token list mode) and its validity
  auto token_row = [&](int e, bool& valid) {
    const int64_t off = rows[e];
    valid = off >= 0;
    return valid ? off : ~off;
  };
  // byte offset of token t of a stage that may straddle pages, and whether
  // its page is valid (a token on an absent page is masked like a token past
  // the stage, and its lane reads row 0 of the sequence instead)
  auto stage_row = [&](int t, bool& valid) {
    const int64_t off = row_offset(kv, b, g, t);
    valid = off >= 0;
    return valid ? off : row0;
  };
  auto issue = [&](int st, StageRegs<D>& R, int& len) {
    len = st_len[wave][st];
    if (len == 0) return;
    const int64_t base = st_base[wave][st];
    R.ok = 0u;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int ti = min(16 * tau + r16, len - 1);
      int64_t off;
      bool valid = true;
      if (tok_list) off = token_row((int)base + ti, valid);
      else if (whole_page) off = base + ti * row_bytes;  // the stage's page is valid
      else off = stage_row((int)base + ti, valid);
      R.ok |= (valid && 16 * tau + r16 < len ? 1u : 0u) << tau;
#pragma unroll
      for (int c = 0; c < KC; ++c)
        R.k[tau][c] = *reinterpret_cast<const uint4*>(kv.k_pool + off + (32 * c + 8 * grp) * EB);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int ti = min(TPV * u + vt, len - 1);
      int64_t off;
      bool valid;
      if (tok_list) off = token_row((int)base + ti, valid);
      else if (whole_page) off = base + ti * row_bytes;
      else off = stage_row((int)base + ti, valid);
      R.v[u] = *reinterpret_cast<const uint4*>(kv.v_pool + off + vd * EB);
    }
  };
  // Fold stage R (len valid tokens) into the online-softmax state.
  auto consume = [&](const StageRegs<D>& R, int len) {
    if (len == 0) return;
    f32x4_t acc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      acc[tau] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c)
        acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            aq[c], __builtin_bit_cast(bf16x8_t, R.k[tau][c]), acc[tau], 0, 0, 0);
    }
    // register i of lane (grp, r16) holds head 4 i + grp
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      const float x0 = (R.ok & 1u) ? acc[0][i] * scale : -INFINITY;
      const float x1 = (R.ok & 2u) ? acc[1][i] * scale : -INFINITY;
      const float mx = group_max<16>(fmaxf(x0, x1));
      const float mn = fmaxf(m_run[i], mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m_run[i] - ms);
      const float p0 = exp2f(x0 - ms), p1 = exp2f(x1 - ms);
      l_run[i] = l_run[i] * alpha + p0 + p1;
      m_run[i] = mn;
      const int j = 4 * i + grp;
      if (j < G) {
        sp[wave][r16][j] = p0;
        sp[wave][16 + r16][j] = p1;
        if (r16 == 0) salpha[wave][j] = alpha;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // p.v on the VALU: lane (vt, vd) accumulates its tokens into dims vd..vd+7
    float al[G];
#pragma unroll
    for (int j = 0; j < G; ++j) al[j] = salpha[wave][j];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) o[j][k] *= al[j];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float vf[8];
      Vec16<bf16_t>::unpack(R.v[u], vf);
      const int tt = TPV * u + vt;
      float pj[G];
#pragma unroll
      for (int j = 0; j < G; ++j) pj[j] = sp[wave][tt][j];
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[j][k] = fmaf(pj[j], vf[k], o[j][k]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Stage table: wave w owns entries e0 + w + 4 i; an entry has ceil(S / 32)
  // stages. One lane per stage looks up the block id and the page and records
  // the stage's first row (byte offset, or its first token when a stage may
  // straddle pages) and its number of valid tokens, so that the pipeline
  // below never waits on a lookup.
  // Token list mode: wave w owns the groups of 32 entries w, w + 4, ...
  const int spe = (S + 31) / 32;
  const int first = e0 + wave;
  const int nent = first < e1 ? (e1 - first + kDecWaves - 1) / kDecWaves : 0;
  const int ngrp = (e1 - e0 + 31) / 32;
  const int nst = tok_list ? (ngrp > wave ? (ngrp - wave + kDecWaves - 1) / kDecWaves : 0)
                           : nent * spe;
  for (int c0 = 0; c0 < nst; c0 += kStagesPerChunk) {
    const int cst = min(kStagesPerChunk, nst - c0);
    if (tok_list && lane < cst) {
      const int pos = e0 + 32 * (wave + kDecWaves * (c0 + lane));  // first list entry
      st_base[wave][lane] = pos;
      st_len[wave][lane] = min(32, e1 - pos);
    } else if (lane < cst) {
      const int st = c0 + lane, i = st / spe, sub = st % spe;
      const int beta = ids[first + kDecWaves * i];
      int64_t base = 0;
      int len = 0;
      if ((unsigned)beta < (unsigned)nb) {
        const int ts = beta * S + 32 * sub, te = min(beta * S + S, T);
        len = max(0, min(32, te - ts));
        if (whole_page && len > 0) {
          const int page = kv.page_table[(int64_t)b * kv.max_pages + ts / kv.page_size];
          if ((unsigned)page < (unsigned)kv.num_phys_pages)
            base = (((int64_t)page * kv.num_kv_heads + g) * kv.page_size + ts % kv.page_size) *
                   row_bytes;
          else
            len = 0;  // absent page: the stage contributes nothing
        } else {
          base = ts;
        }
      }
      st_base[wave][lane] = base;
      st_len[wave][lane] = len;
    }
    __builtin_amdgcn_wave_barrier();
    // two-deep software pipeline: stage s + 1 is loading while s computes
    StageRegs<D> A, B;
    int lenA = 0, lenB = 0;
    issue(0, A, lenA);
    for (int st = 0; st < cst; st += 2) {
      if (st + 1 < cst) issue(st + 1, B, lenB);
      consume(A, lenA);
      if (st + 1 >= cst) break;
      if (st + 2 < cst) issue(st + 2, A, lenA);
      consume(B, lenB);
    }
    __builtin_amdgcn_wave_barrier();
  }
  // the running max is uniform per head across the wave, so the token groups'
  // partial sums add without rescaling
#pragma unroll
  for (int s = VL; s < kWave; s *= 2)
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) o[j][k] += __shfl_xor(o[j][k], s);
#pragma unroll
  for (int i = 0; i < GR; ++i) l_run[i] = group_sum<16>(l_run[i]);
  if (lane < VL) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) sh.o[wave][j][vd + k] = o[j][k];
  }
  if (r16 == 0) {
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      const int j = 4 * i + grp;
      if (j < G) {
        sh.m[wave][j] = m_run[i];
        sh.l[wave][j] = l_run[i];
      }
    }
  }
}

// -------------------------------------------------------------- float32 path
// Attention over ids[e0 .. e1) for a float32 cache; leaves each wave's state
// in ds.sh for finish_split.
template <int D, int G, int UNR>
__device__ __forceinline__ void attend_f32(const DecodeParams& p, int unit, const int32_t* ids,
                                           int e0, int e1, DecodeShared<D, G>& ds) {
  constexpr int EPL = 4;              // floats per 16-byte load
  constexpr int LPT = D / EPL;        // lanes per token row
  constexpr int TPW = kWave / LPT;    // tokens per wave instruction
  SplitShared<D, G>& sh = ds.sh;
  const KvView& kv = p.kv;
  const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
  const int T = clamp_len(kv, b);
  const int S = p.block_size;
  const int nb = (T + S - 1) / S;
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  const int tg = lane / LPT, li = lane % LPT;
  const int Hq = kv.num_kv_heads * G;

  float qv[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float4 r = *reinterpret_cast<const float4*>(
        reinterpret_cast<const float*>(p.q) + ((int64_t)b * Hq + g * G + j) * D + li * EPL);
    qv[j][0] = r.x * p.scale_log2;
    qv[j][1] = r.y * p.scale_log2;
    qv[j][2] = r.z * p.scale_log2;
    qv[j][3] = r.w * p.scale_log2;
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[j][k] = 0.f;
  }
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
        Vec16<float>::unpack(kr[u], kf);
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
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float alpha = exp2f(m[j] - ms);
        m[j] = mn;
        l[j] *= alpha;
#pragma unroll
        for (int k = 0; k < EPL; ++k) o[j][k] *= alpha;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          pr[u][j] = exp2f(x[u][j] - ms);
          l[j] += pr[u][j];
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float vf[EPL];
        Vec16<float>::unpack(vr[u], vf);
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int k = 0; k < EPL; ++k) o[j][k] = fmaf(pr[u][j], vf[k], o[j][k]);
      }
    }
  }
  // merge the token groups of the wave (their running maxima differ)
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
  if (tg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) sh.o[wave][j][li * EPL + k] = o[j][k];
      if (li == 0) {
        sh.m[wave][j] = m[j];
        sh.l[wave][j] = l[j];
      }
    }
  }
}

// Unroll of the float32 path's token loop (registers bound it at G = 8).
template <int G>
constexpr int f32_unroll() { return G == 8 ? 4 : 8; }

// Attention of one split task over ids[e0 .. e1), then its partial and
// arrival (the last task of the unit merges).
// TOK: single tokens given by their row offsets rows[e0 .. e1) (block size
// 1; see attend_bf16).
template <typename TE, int D, int G, bool TOK = false>
__device__ __forceinline__ void decode_split(const DecodeParams& p, int unit, int split,
                                             const int32_t* ids, int e0, int e1,
                                             DecodeShared<D, G>& ds,
                                             const int64_t* rows = nullptr) {
  if constexpr (sizeof(TE) == 2) attend_bf16<D, G, TOK>(p, unit, ids, e0, e1, ds, rows);
  else attend_f32<D, G, f32_unroll<G>()>(p, unit, ids, e0, e1, ds);
  finish_split<D, G>(p, ds.sh, unit, split);
}

}  // namespace
}  // namespace hs
