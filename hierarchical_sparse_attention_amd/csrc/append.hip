// append.hip - decode-time cache maintenance: one new token per sequence is
// written into its page slot and the sequence length advanced on the device.
//
// Sources: "SGLang hierarchical sparse attention: analysis and practice",
// section 2.2 (each decode step appends the new token's K/V to the paged
// cache, addressed through the logical -> physical page table); untitled
// HiSparse project write-up, section 3.1 (the per-block table lives in HBM
// and is updated as the cache is written: the summary refresh of the growing
// block is hs_build_summaries / hs_decode_step with a block_begin).
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kAppendThreads = 256;

// One workgroup per sequence b: t = seq_lens[b]; if t is inside the cache's
// capacity and its page id is valid, the rows k_new[b][g] and v_new[b][g] of
// every KV head g are copied (16-byte chunks) to slot t % P of page
// page_table[b][t / P], then seq_lens[b] = t + 1. Otherwise nothing changes.
__global__ __launch_bounds__(kAppendThreads) void k_append(AppendParams p) {
  const KvView& kv = p.kv;
  const int b = blockIdx.x;
  const int t = p.seq_lens[b];  // every thread reads it before the barrier below
  const bool ok = t >= 0 && t < kv.max_seq_len && row_offset(kv, b, 0, t) >= 0;
  const int row_chunks = kv.head_dim * kv.elem_bytes / 16;  // 16-byte chunks per row
  const int chunks = kv.num_kv_heads * row_chunks;          // per pool
  if (ok) {
    for (int i = thread_id(); i < 2 * chunks; i += kAppendThreads) {
      const bool is_v = i >= chunks;
      const int j = is_v ? i - chunks : i;
      const int g = j / row_chunks, c = j % row_chunks;
      const int64_t src = ((int64_t)b * kv.num_kv_heads + g) * row_chunks + c;
      const uint4 x = reinterpret_cast<const uint4*>(is_v ? p.v_new : p.k_new)[src];
      uint8_t* pool = is_v ? p.v_pool : p.k_pool;
      *reinterpret_cast<uint4*>(pool + row_offset(kv, b, g, t) + (int64_t)c * 16) = x;
    }
  }
  __syncthreads();  // every thread has read seq_lens[b]
  if (ok && thread_id() == 0) p.seq_lens[b] = t + 1;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_append, dim3(p.kv.batch), dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs
