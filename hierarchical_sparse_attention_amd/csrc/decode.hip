// decode.hip - stage 3 as one launch: grid (n_splits, units), one split task
// per workgroup; the unit's last task merges. The device code and its
// sources are in decode_impl.h.
#include "decode_impl.h"

namespace hs {
namespace {

constexpr int kTargetTasks = 256;         // compute units of the GPU: about one split task each
constexpr int64_t kLongSplit = 2048;      // tokens per split (full selection) that double the splits

// One split task: the unit's count is read, its run of ids is copied into LDS
// (written by an earlier launch, so plain loads), then attention and merge.
// TOK: block size 1, the ids are a token list (bf16 caches; the float32 path
// handles any block size as it is); every token's page is looked up here, in
// one pass over the run, and LDS holds the rows' byte offsets, so that the
// attention's loads never wait on a lookup.
template <typename TE, int D, int G, bool TOK>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeParams p) {
  __shared__ DecodeShared<D, G> ds;
  extern __shared__ int64_t dyn_lds[];  // the run: int32 ids, or (TOK) int64 row offsets
  const int unit = blockIdx.y, split = blockIdx.x;
  int cnt = p.counts[unit];
  cnt = cnt < 0 ? 0 : (cnt > p.max_selected ? p.max_selected : cnt);
  int e0, e1;
  split_range(cnt, p.n_splits, split, e0, e1);
  const int32_t* ids = p.ids + (int64_t)unit * p.max_selected;
  if constexpr (TOK) {
    const KvView& kv = p.kv;
    const int b = unit / kv.num_kv_heads, g = unit % kv.num_kv_heads;
    const int T = clamp_len(kv, b);
    // a masked token (outside [0, T) or on an absent page) is stored as ~r,
    // r the offset of row 0 of the sequence (finite values), which its lane
    // reads instead; its page is looked up here, beside the list's
    const int64_t r0 = T > 0 ? max(row_offset(kv, b, g, 0), (int64_t)0) : 0;
    int64_t* rows = dyn_lds;
    for (int i = thread_id(); i < e1 - e0; i += kDecThreads) {
      const int t = ids[e0 + i];
      const int64_t off = (unsigned)t < (unsigned)T ? row_offset(kv, b, g, t) : -1;
      rows[i] = off >= 0 ? off : ~r0;
    }
    __syncthreads();
    decode_split<TE, D, G, true>(p, unit, split, nullptr, 0, e1 - e0, ds, rows);
  } else {
    int32_t* run = reinterpret_cast<int32_t*>(dyn_lds);
    for (int i = thread_id(); i < e1 - e0; i += kDecThreads) run[i] = ids[e0 + i];
    __syncthreads();
    decode_split<TE, D, G, false>(p, unit, split, run, 0, e1 - e0, ds);
  }
}

static_assert(sizeof(DecodeShared<128, 8>) + kDecodeRunLds <= (160u << 10),
              "a split task's LDS fits a compute unit's 160 KiB");

template <typename TE, int D, int G, bool TOK>
hipError_t launch_one(const DecodeParams& p, dim3 grid, size_t lds, hipStream_t s) {
  if (lds + sizeof(DecodeShared<D, G>) > (64u << 10)) {  // above the default LDS limit
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<TE, D, G, TOK>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_decode<TE, D, G, TOK>), grid, dim3(kDecThreads), lds, s, p);
  return hipGetLastError();
}

template <typename TE, int D, bool TOK>
hipError_t launch_g(const DecodeParams& p, dim3 grid, size_t lds, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_one<TE, D, 1, TOK>(p, grid, lds, s);
    case 2: return launch_one<TE, D, 2, TOK>(p, grid, lds, s);
    case 4: return launch_one<TE, D, 4, TOK>(p, grid, lds, s);
    default: return launch_one<TE, D, 8, TOK>(p, grid, lds, s);
  }
}

template <int D>
hipError_t launch_bf16(const DecodeParams& p, dim3 grid, size_t lds, hipStream_t s) {
  return p.block_size == 1 ? launch_g<bf16_t, D, true>(p, grid, lds, s)
                           : launch_g<bf16_t, D, false>(p, grid, lds, s);
}

}  // namespace

int decode_splits(int64_t units, int32_t max_selected, int32_t block_size) {
  int64_t ns = (kTargetTasks + units - 1) / units;
  if ((int64_t)max_selected * block_size >= kLongSplit * ns) ns = (2 * kTargetTasks + units - 1) / units;
  if (ns > max_selected) ns = max_selected;
  if (ns > kMaxSplits) ns = kMaxSplits;
  return ns < 1 ? 1 : (int)ns;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.n_splits, p.kv.batch * p.kv.num_kv_heads);
  const size_t lds = decode_run_bytes(p.kv.elem_bytes, p.block_size, p.max_selected, p.n_splits);
  if (p.kv.elem_bytes == 2)
    return p.kv.head_dim == 64 ? launch_bf16<64>(p, grid, lds, s) : launch_bf16<128>(p, grid, lds, s);
  return p.kv.head_dim == 64 ? launch_g<float, 64, false>(p, grid, lds, s)
                             : launch_g<float, 128, false>(p, grid, lds, s);
}

}  // namespace hs
