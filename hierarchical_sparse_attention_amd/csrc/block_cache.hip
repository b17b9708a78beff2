// block_cache.hip - LRU cache of selected blocks and the step difference.
//
// Source: "SGLang hierarchical sparse attention: analysis and practice",
// section 3.2 (the sparse diff kernel): consecutive steps select largely the
// same blocks; a cache pool a few times the top-k is kept least-recently-used;
// each step takes the difference from the previous selection, finds the
// cached blocks (hits), loads the misses and updates the cache index. Without
// a host tier the cache is its index: per unit, `capacity` slots of (block id,
// step of last selection).
//
// Rule (unique result): at step t every selected block found in a slot is a
// hit and gets stamp t; the misses, in ascending block order, take the slots
// not hit at this step ordered by (stamp, slot index), empty slots (stamp -1)
// first; the step difference counts selected blocks whose slot did not carry
// stamp t - 1.
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kCacheThreads = 256;
constexpr int32_t kHitKey = 0x7FFFFFFF;  // eviction key of a slot hit at this step

__device__ __forceinline__ uint32_t wg_excl_sum(uint32_t x, uint32_t* tot, uint32_t* total) {
  const int tid = thread_id(), lane = tid & (kWave - 1), wave = tid / kWave;
  uint32_t inc = x;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    inc += lane >= d ? y : 0u;
  }
  if (lane == kWave - 1) tot[wave] = inc;
  __syncthreads();
  uint32_t off = 0, all = 0;
  for (int w = 0; w < kCacheThreads / kWave; ++w) {
    off += w < wave ? tot[w] : 0u;
    all += tot[w];
  }
  *total = all;
  return off + inc - x;
}

// One workgroup per unit. Dynamic LDS: ids, slot of each id, "stamp was t-1"
// flags and the miss order (max_selected each), then the slots' eviction keys
// (capacity).
__global__ __launch_bounds__(kCacheThreads) void k_cache_update(CacheParams p) {
  extern __shared__ int32_t lds[];
  __shared__ uint32_t tot[kCacheThreads / kWave];
  __shared__ uint32_t misses_total, prev_total;
  const int M = p.max_selected, C = p.capacity, t = p.step;
  int32_t* ids = lds;
  int32_t* sof = ids + M;
  int32_t* prevf = sof + M;
  int32_t* mj = prevf + M;
  int32_t* ekey = mj + M;
  const int u = blockIdx.x, tid = thread_id();
  int cnt = p.counts[u];
  cnt = cnt < 0 ? 0 : (cnt > M ? M : cnt);
  int32_t* sblk = p.slot_block + (int64_t)u * C;
  int32_t* sst = p.slot_stamp + (int64_t)u * C;
  for (int j = tid; j < cnt; j += kCacheThreads) {
    ids[j] = p.ids[(int64_t)u * M + j];
    sof[j] = -1;
    prevf[j] = 0;
  }
  __syncthreads();
  // hits: each slot's block is looked up in the ascending ids (binary search)
  for (int s = tid; s < C; s += kCacheThreads) {
    const int32_t b = sblk[s], st = sst[s];
    int lo = 0, hi = cnt;  // first index with ids[idx] >= b
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ids[mid] < b) lo = mid + 1;
      else hi = mid;
    }
    const bool hit = b >= 0 && lo < cnt && ids[lo] == b;
    if (hit) {
      sof[lo] = s;
      prevf[lo] = st == t - 1 ? 1 : 0;
    }
    ekey[s] = hit ? kHitKey : st;
  }
  __syncthreads();
  // misses numbered in ascending id order (each thread a contiguous range)
  const int per = (cnt + kCacheThreads - 1) / kCacheThreads;
  const int j0 = min(cnt, tid * per), j1 = min(cnt, j0 + per);
  uint32_t mine = 0, prev = 0;
  for (int j = j0; j < j1; ++j) {
    mine += sof[j] < 0 ? 1u : 0u;
    prev += (uint32_t)prevf[j];
  }
  uint32_t n_miss;
  uint32_t r = wg_excl_sum(mine, tot, &n_miss);
  for (int j = j0; j < j1; ++j)
    if (sof[j] < 0) mj[r++] = j;
  __syncthreads();  // tot is reused below
  uint32_t n_prev;
  wg_excl_sum(prev, tot, &n_prev);
  if (tid == 0) {
    misses_total = n_miss;
    prev_total = n_prev;
  }
  __syncthreads();  // mj complete
  // victims: slot s not hit at this step takes miss number rank(s), its place
  // in (stamp, slot) order among those slots
  for (int s = tid; s < C; s += kCacheThreads) {
    const int32_t k = ekey[s];
    if (k == kHitKey) {
      sst[s] = t;
      continue;
    }
    uint32_t rank = 0;
    if (n_miss > 0)
      for (int s2 = 0; s2 < C; ++s2) {
        const int32_t k2 = ekey[s2];
        rank += (k2 < k || (k2 == k && s2 < s)) ? 1u : 0u;
      }
    if (rank < n_miss) {
      const int j = mj[rank];
      sof[j] = s;
      sblk[s] = ids[j];
      sst[s] = t;
    }
  }
  __syncthreads();  // sof complete
  for (int j = tid; j < cnt; j += kCacheThreads) p.slot_of[(int64_t)u * M + j] = sof[j];
  for (int q = tid; q < (int)n_miss; q += kCacheThreads)
    p.miss_blocks[(int64_t)u * M + q] = ids[mj[q]];
  if (tid == 0) {
    p.stats[3 * u + 0] = cnt - (int)misses_total;
    p.stats[3 * u + 1] = (int)misses_total;
    p.stats[3 * u + 2] = cnt - (int)prev_total;
  }
}

}  // namespace

size_t cache_lds_bytes(int32_t max_selected, int32_t capacity) {
  return sizeof(int32_t) * (4 * (size_t)max_selected + capacity);
}

hipError_t launch_cache_update(const CacheParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_cache_update, dim3(p.units), dim3(kCacheThreads),
                     cache_lds_bytes(p.max_selected, p.capacity), s, p);
  return hipGetLastError();
}

}  // namespace hs
