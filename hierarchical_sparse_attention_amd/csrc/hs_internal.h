// hs_internal.h - device helpers and kernel-launch declarations shared by the
// HIP sources of libhs_attn.so (gfx950 / CDNA4, wave64). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_attn.h"

namespace hs {

constexpr int kWave = 64;

// Thread index in the workgroup, read through an empty asm: every call is a
// new value to the compiler. Task bodies take it once at their start, so in
// a persistent task loop the per-thread address arithmetic of a task is
// recomputed per task instead of being hoisted out of the loop, where it
// would hold registers for the whole kernel.
__device__ __forceinline__ int thread_id() {
  int x = threadIdx.x;
  asm volatile("" : "+v"(x));
  return x;
}

// ----------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 16 bytes of storage -> EPL floats (EPL = 4 for float32, 8 for bfloat16).
template <typename TE>
struct Vec16;

template <>
struct Vec16<float> {
  static constexpr int EPL = 4;
  __device__ __forceinline__ static void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};

struct bf16_t {
  uint16_t bits;
};

template <>
struct Vec16<bf16_t> {
  static constexpr int EPL = 8;
  __device__ __forceinline__ static void unpack(const uint4& r, float* f) {
    f[0] = bf16_lo(r.x);
    f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y);
    f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z);
    f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w);
    f[7] = bf16_hi(r.w);
  }
};

// Monotone map of a float32 to uint32: a < b (as floats, -0 == +0) iff
// key(a) < key(b). Negative values have all bits flipped, non-negative ones
// only the sign bit; -0 is mapped like +0. Finite inputs give keys >= 0x00800000.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Score stored for a candidate slot that holds no block: the all-ones NaN,
// whose key is 0, the key of "no candidate".
constexpr uint32_t kAbsentScore = 0xFFFFFFFFu;

// ------------------------------------------------------ cross-lane reduction
// Sum over aligned groups of N lanes (N in {1, 2, 4, 8, 16, 32, 64}); every
// lane of a group ends with the group's sum. Within a 16-lane DPP row the
// butterfly uses quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and
// row_mirror (after the two quad steps every lane of a quad holds the quad's
// sum, so the mirrors pair whole quads, then whole half-rows); wider groups
// exchange with the lanes 16 and 32 apart.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// ------------------------------------------- cross-workgroup hand-off
// Data that another workgroup of the same launch reads (split partials,
// block scores) is written and read with relaxed device-scope atomic accesses:
// on gfx950 they are plain loads and stores with the sc1 bit, which makes them
// coherent across the per-XCD L2 caches without writing back or invalidating
// a whole L2 (what a device-scope fence costs). A workgroup drains its stores
// (s_waitcnt vmcnt(0)) and synchronises before one lane increments the
// arrival counter; the workgroup that sees the last arrival then reads the
// published data with device-scope loads.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float published(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_i32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t published_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Arrival counters and flags that workgroups poll or update live one per
// 256-byte line (kCounterStride int32s apart), so that pollers of different
// units hit different memory channels.
constexpr int kCounterStride = 64;
__device__ __forceinline__ int32_t* counter_of(int32_t* base, int unit) {
  return base + (int64_t)unit * kCounterStride;
}

// Every thread calls this; returns true in every thread of the workgroup that
// arrived last (of `expected`) on `counter`, which it then resets to zero.
__device__ __forceinline__ bool arrive_last(int32_t* counter, int expected, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's published stores are done
  __syncthreads();
  if (thread_id() == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == expected - 1;
    if (*flag) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag;
}

// ------------------------------------------------------------- cache access
struct KvView {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t batch, num_kv_heads, head_dim, page_size, max_pages, num_phys_pages, max_seq_len;
  int32_t elem_bytes;
};

__device__ __forceinline__ int clamp_len(const KvView& kv, int b) {
  int t = kv.seq_lens[b];
  t = t < 0 ? 0 : t;
  return t > kv.max_seq_len ? kv.max_seq_len : t;
}

// Byte offset of row (b, g, t) in a pool, or -1 if its page id is invalid.
__device__ __forceinline__ int64_t row_offset(const KvView& kv, int b, int g, int t) {
  int page = kv.page_table[(int64_t)b * kv.max_pages + t / kv.page_size];
  if ((unsigned)page >= (unsigned)kv.num_phys_pages) return -1;
  return (((int64_t)page * kv.num_kv_heads + g) * kv.page_size + t % kv.page_size) *
         (int64_t)kv.head_dim * kv.elem_bytes;
}

// -------------------------------------------------------- launch interfaces
struct SummParams {
  KvView kv;
  void* out;
  int32_t kind, block_size, max_blocks, block_begin;
};
hipError_t launch_build_summaries(const SummParams& p, hipStream_t s);

// Decode-time append of one token per sequence.
struct AppendParams {
  KvView kv;                 // shapes, page table (its pools are the ones written)
  uint8_t* k_pool;
  uint8_t* v_pool;
  const void* k_new;         // [B][Hkv][d] in the cache dtype
  const void* v_new;
  int32_t* seq_lens;         // [B] read, advanced by one where the token was written
};
hipError_t launch_append(const AppendParams& p, hipStream_t s);

// LRU cache of selected blocks: one step of every unit.
struct CacheParams {
  int32_t* slot_block;       // [units][capacity]
  int32_t* slot_stamp;       // [units][capacity]
  int32_t capacity;
  int32_t units, step, max_selected;
  const int32_t* ids;        // [units][max_selected] ascending
  const int32_t* counts;     // [units]
  int32_t* slot_of;          // [units][max_selected]
  int32_t* miss_blocks;      // [units][max_selected]
  int32_t* stats;            // [units][3]: hits, misses, step difference
};
constexpr int kMaxCacheSlots = 1024;
constexpr int kMaxCacheSelected = 2048;
hipError_t launch_cache_update(const CacheParams& p, hipStream_t s);

// Selection-level kind beyond the public summary kinds: the candidates are
// single tokens (block size 1) whose "summary rows" are their K rows, read
// through the page table (the token-level second stage).
constexpr int32_t kKindTokens = 2;

// One selection level (fused scoring + top-k + window).
struct SelectParams {
  KvView kv;                 // shapes + seq_lens
  const void* q;             // [B][Hq][d]
  const void* summ;          // summary table of this level
  int32_t kind, block_size, max_blocks;
  int32_t G;
  // candidate slots: single level -> slot c is block c (n_slots = ceil(T_b/S));
  // two-level fine -> slot c is block gamma[c / R] * R + c % R.
  const int32_t* gamma;      // [units][gamma_cap] ascending coarse ids, or null
  const int32_t* gamma_cnt;  // [units]
  int32_t gamma_cap, ratio;  // R = C / S
  int32_t n_slots_max;       // scores row length
  float* scores;             // [units][n_slots_max]
  uint32_t* chunk_keys;      // [units][chunks][2]: largest order key, largest ~key of a chunk
  int32_t top_k;
  float top_k_ratio;         // > 0: k = max(1, int(nb * ratio)) per unit instead of top_k
  const int32_t* forced;     // [units][forced_cap] block ids unioned in, or null
  int32_t forced_cap;
  int32_t window;            // tokens (0 = none)
  int32_t* out_ids;          // [units][out_cap]
  int32_t* out_cnt;          // [units]
  int32_t out_cap;
  int32_t out_blocks_max;    // blocks of this level per unit (bitmap bits)
  int32_t* counters;         // [units] workgroup arrivals; zero between calls
  int32_t refresh_begin;     // >= 0: rebuild blocks from here on before scoring (single level)
  // With refresh_begin >= 0: when set, another workgroup of the launch
  // rebuilds those blocks and then counts itself on the unit's word
  // rebuilt_by + unit * kCounterStride; the scoring waits for that arrival
  // (bounded by wait_ticks, an expiry recorded in *status) and takes it off
  // again, so the word is zero between calls whatever the order.
  int32_t* rebuilt_by = nullptr;
  int32_t* status = nullptr;
  long long wait_ticks = 0;
};
hipError_t launch_select(const SelectParams& p, hipStream_t s);

// Head of a two-level decode step, one launch of two workgroups per unit:
// the first rebuilds the coarse table's blocks from coarse_begin (the whole
// workgroup each), then the fine table's blocks from fine_begin (one wave
// each); the second scores the unit's coarse rows meanwhile, rescores the
// rebuilt ones once the first has stored them, and runs the coarse
// selection. `coarse` holds the coarse level's selection parameters (its
// table is coarse.summ, of mean summaries, and its candidates fit one
// scoring chunk).
struct HeadParams {
  void* fine;  // fine summary table
  int32_t fine_kind, fine_block, fine_max_blocks, fine_begin;
  int32_t coarse_begin;
  int32_t* status;  // the step's status word (HS_STEP_WAIT_EXPIRED on an expired wait)
};
bool two_level_head_fits(const SelectParams& coarse, int32_t fine_block, int32_t coarse_kind);
hipError_t launch_two_level_head(const SelectParams& coarse, const HeadParams& h, hipStream_t s);
// Dynamic LDS of a selection workgroup: bitmap words, then keys (general path).
size_t select_lds_bytes(int32_t out_blocks_max, int32_t n_slots_max);
// Total dynamic LDS of a k_select launch (adds the staged id list).
size_t select_launch_lds_bytes(int32_t out_blocks_max, int32_t n_slots_max, int32_t out_cap);
// Whether a selection of this kind and size takes the token level's register
// path, which needs no dynamic LDS (no bitmap, no staged list).
bool tokens_in_registers(int32_t kind, int32_t n_slots_max, int32_t gamma_cap);

struct DecodeParams {
  KvView kv;
  const void* q;
  int32_t G;
  float scale_log2;          // scale * log2(e)
  int32_t block_size;
  const int32_t* ids;        // [units][max_selected] (separate launch)
  const int32_t* counts;     // [units]
  int32_t max_selected;
  int32_t n_splits;          // split tasks per unit (<= kMaxSplits)
  float* part_o;             // [units][n_splits][G][d]
  float* part_ml;            // [units][n_splits][G][2]
  int32_t* counters;         // [units] split arrivals; zero between calls
  int32_t* score_counters;   // fused launch: [units] scoring arrivals to clear, else null
  int32_t score_chunks;      // fused launch: scoring arrivals per unit
  float* out;                // [B][Hq][d]
};
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
constexpr int kMaxSplits = 128;
// Split tasks per unit: enough to give every compute unit of the GPU about
// one task (the work of a unit is its id list), two when a split would still
// hold many tokens at the full selection (a second resident workgroup per
// compute unit keeps more KV loads in flight), at most one per selectable
// block and at most kMaxSplits.
int decode_splits(int64_t units, int32_t max_selected, int32_t block_size);
// LDS of the run of the list that one split task of the separate decode
// launch holds: int32 ids, or int64 row offsets for the token lists (block
// size 1) of a bf16 cache; larger runs are refused before the launch.
constexpr size_t kDecodeRunLds = 96u << 10;
inline size_t decode_run_bytes(int elem_bytes, int32_t block_size, int32_t max_selected,
                               int n_splits) {
  const size_t per = elem_bytes == 2 && block_size == 1 ? sizeof(int64_t) : sizeof(int32_t);
  return per * (size_t)((max_selected + n_splits - 1) / n_splits);
}

// Control line of the fused launch at the start of its workspace (int32
// index of the status word the host reads; the line is 256 bytes).
constexpr int kCtrlStatus = 0;
constexpr int kCtrlBytes = kCounterStride * 4;

// Fused last selection level + decode of one layer (one persistent launch).
struct StepParams {
  SelectParams sel;          // the last (or only) selection level
  DecodeParams dec;          // counts / out / workspace of the decode
  int32_t units, n_chunks, total;
  int32_t list_cap;          // LDS id list entries (= sel.out_cap)
  int32_t* ctrl;             // control line (kCtrlStatus)
  long long wait_ticks;      // bound of a wait, in wall-clock ticks (set by launch_step)
};
hipError_t launch_step(const StepParams& p, hipStream_t s);
// Bound of a wait on another workgroup of a launch, in wall-clock ticks of
// the current device (a quarter of a second).
hipError_t wait_bound(long long* ticks);
int step_chunks(int32_t n_slots_max);  // scoring tasks per unit
// Whether the fused kernel's LDS (bitmap, keys, id list) fits for these sizes.
bool step_fits(int32_t out_blocks_max, int32_t n_slots_max, int32_t list_cap);

constexpr int kMaxBlocks = 32768;  // blocks per unit of a summary level (LDS bitmap)

}  // namespace hs
