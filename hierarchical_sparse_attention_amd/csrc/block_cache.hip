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

constexpr int kCacheThreads = 1024;  // one slot (capacity <= 1024) and one sort pair per thread
constexpr int kMaxClasses = 8;       // stamp classes taken one by one before sorting

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

// Slots are ordered for eviction by the 64-bit key (stamp + 1, slot index):
// empty slots (stamp -1) first, then least recently used, ties by index.
// Slots hit at this step, and the padding up to a power of two, sort last.
__host__ __device__ inline int sort_size(int c) {
  int n = 1;
  while (n < c) n <<= 1;
  return n;
}

// One workgroup per unit. Dynamic LDS: ids, slot of each id, "stamp was t-1"
// flags and the miss order (max_selected each), then the eviction keys
// (sort_size(capacity) 64-bit words, 8-byte aligned).
__global__ __launch_bounds__(kCacheThreads) void k_cache_update(CacheParams p) {
  extern __shared__ int32_t lds[];
  __shared__ uint32_t tot[kCacheThreads / kWave];
  __shared__ uint32_t cls_min[kCacheThreads / kWave];
  const int M = p.max_selected, C = p.capacity, t = p.step;
  const int N = sort_size(C);
  int32_t* ids = lds;
  int32_t* sof = ids + M;
  int32_t* prevf = sof + M;
  int32_t* mj = prevf + M;
  uint64_t* key = reinterpret_cast<uint64_t*>(mj + M);  // 16 * M bytes in: 8-byte aligned
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
  for (int s = tid; s < N; s += kCacheThreads) {
    uint64_t k = ~0ull;
    if (s < C) {
      const int32_t b = sblk[s], st = sst[s];
      int lo = 0, hi = cnt;  // first index with ids[idx] >= b
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ids[mid] < b) lo = mid + 1;
        else hi = mid;
      }
      if (b >= 0 && lo < cnt && ids[lo] == b) {
        sof[lo] = s;
        prevf[lo] = st == t - 1 ? 1 : 0;
        sst[s] = t;
      } else {
        k = ((uint64_t)(uint32_t)(st + 1) << 32) | (uint32_t)s;
      }
    }
    key[s] = k;
  }
  __syncthreads();
  // misses numbered in ascending id order (each thread a contiguous range),
  // and the count of selected blocks that carried stamp t - 1
  const int per = (cnt + kCacheThreads - 1) / kCacheThreads;
  const int j0 = min(cnt, tid * per), j1 = min(cnt, j0 + per);
  uint32_t mine = 0, prev = 0;
  for (int j = j0; j < j1; ++j) {
    mine += sof[j] < 0 ? 1u : 0u;
    prev += (uint32_t)prevf[j];
  }
  uint32_t n_miss, n_prev;
  uint32_t r = wg_excl_sum(mine, tot, &n_miss);
  for (int j = j0; j < j1; ++j)
    if (sof[j] < 0) mj[r++] = j;
  __syncthreads();  // tot is reused
  wg_excl_sum(prev, tot, &n_prev);
  // Eviction order. The misses usually fit in the few oldest stamp classes:
  // classes are taken one at a time (the workgroup's smallest remaining
  // stamp, then a prefix sum in slot order, slot s being thread s), which is
  // exactly the start of the (stamp, slot) order. Past kMaxClasses classes
  // the keys are sorted instead and the order continues from there.
  uint32_t base = 0;  // misses placed so far
  {
    const uint64_t mykey = tid < N ? key[tid] : ~0ull;
    const bool elig = mykey != ~0ull;
    const uint32_t myst = (uint32_t)(mykey >> 32);  // stamp + 1
    uint32_t floor_st = 0;                          // classes below it are taken
    for (int cls = 0; base < n_miss && cls < kMaxClasses; ++cls) {  // uniform
      uint32_t v = elig && myst >= floor_st ? myst : 0xFFFFFFFFu;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d));
      if ((tid & (kWave - 1)) == 0) cls_min[tid / kWave] = v;
      __syncthreads();
      uint32_t m = 0xFFFFFFFFu;
      for (int w = 0; w < kCacheThreads / kWave; ++w) m = min(m, cls_min[w]);
      if (m == 0xFFFFFFFFu) break;  // no eligible slot left (uniform)
      const bool in = elig && myst == m;
      uint32_t n_in;
      const uint32_t r = wg_excl_sum(in ? 1u : 0u, tot, &n_in);
      if (in && base + r < n_miss) {
        const int j = mj[base + r];
        sof[j] = tid;
        sblk[tid] = ids[j];
        sst[tid] = t;
      }
      base += min(n_in, n_miss - base);
      floor_st = m + 1;
      __syncthreads();  // cls_min and tot are rewritten by the next class
    }
  }
  if (base < n_miss) {  // uniform: sort the keys for the rest of the order
    for (int k = 2; k <= N; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < N; i += kCacheThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t a = key[i], b = key[ixj];
            const bool up = (i & k) == 0;
            if ((a > b) == up) {
              key[i] = b;
              key[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
  }
  // miss number q takes the q-th slot of the order (the first `base` are placed)
  for (int q = (int)base + tid; q < (int)n_miss; q += kCacheThreads) {
    const int s = (int)(uint32_t)key[q];
    const int j = mj[q];
    sof[j] = s;
    sblk[s] = ids[j];
    sst[s] = t;
  }
  __syncthreads();  // sof complete
  for (int j = tid; j < cnt; j += kCacheThreads) p.slot_of[(int64_t)u * M + j] = sof[j];
  for (int q = tid; q < (int)n_miss; q += kCacheThreads)
    p.miss_blocks[(int64_t)u * M + q] = ids[mj[q]];
  if (tid == 0) {
    p.stats[3 * u + 0] = cnt - (int)n_miss;
    p.stats[3 * u + 1] = (int)n_miss;
    p.stats[3 * u + 2] = cnt - (int)n_prev;
  }
}

}  // namespace

size_t cache_lds_bytes(int32_t max_selected, int32_t capacity) {
  return sizeof(int32_t) * 4 * (size_t)max_selected + sizeof(uint64_t) * (size_t)sort_size(capacity);
}

hipError_t launch_cache_update(const CacheParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_cache_update, dim3(p.units), dim3(kCacheThreads),
                     cache_lds_bytes(p.max_selected, p.capacity), s, p);
  return hipGetLastError();
}

}  // namespace hs
