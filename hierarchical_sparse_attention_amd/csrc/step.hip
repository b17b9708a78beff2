// step.hip - one decode step of one layer in a single launch: the last
// selection level of stage 2 (scoring, top-k, window) and the sparse
// attention of stage 3 over the ids it selects.
//
// Sources: the same passages as select_impl.h and decode_impl.h; fusing the
// two stages is a scheduling choice of this library, the pages run them as
// separate steps ("8x256K ... porting HiSparse to QSA", section 3.2 then
// section 3.3).
//
// Why one launch: a unit's selection and its attention are a chain of short
// latency-bound phases (scores -> top-k -> page lookups -> KV stream ->
// merge). As separate launches every phase waits for the slowest unit and
// each launch pays its own ramp-up and drain.
//
// Tasks: the U * NC scoring tasks (unit t / NC, chunk t % NC) come first,
// then the U * NS split tasks (unit, split). A scoring task publishes its
// chunk's scores and counts itself on the unit's scoring counter. Every
// split task of a unit waits for that counter to reach NC, then runs the
// unit's whole top-k itself from the published scores into an LDS id list:
// the NS copies of the selection are identical (same scores, same code), so
// no id list or ready flag has to travel between workgroups, which would
// cost three more round trips to the device-coherent level. Split 0 also
// writes the ids and the count to the caller's buffers. Each task then
// attends over its run of the list and publishes a partial; the unit's last
// task merges and clears the unit's counters.
//
// Scheduling: a persistent grid of R workgroups, R = what the GPU holds at
// once (occupancy x compute units, from the HIP occupancy query), so that
// normally every workgroup of the grid is resident together. Task t goes to
// workgroup t % R, which runs its tasks in increasing t. A split task only
// waits for scoring tasks, which have smaller t and never wait: each is done
// or being run by its resident workgroup, whose earlier tasks are scoring
// tasks too, so every wait ends. That needs the whole grid resident: when
// another kernel holds part of the GPU, a workgroup whose scoring task waits
// for a free slot can keep a split task waiting. The wait is therefore
// bounded by wall-clock time; when it expires the task goes on with whatever
// scores are in memory (ids are range-checked, so every access stays in
// bounds), the kernel ends, and the workspace's status word records it for
// the caller. (Handing tasks out through a shared ticket counter would make
// every wait end whatever the residency, but its same-address atomics made
// the 128K step about 9 us slower.)
#include "decode_impl.h"
#include "select_impl.h"

namespace hs {
namespace {

constexpr size_t kMaxDynLds = 48 << 10;  // bitmap + keys + id list

template <int D, int G>
union StepShared {
  TopkShared t;
  DecodeShared<D, G> d;
};

// dynamic LDS words: [bitmap][keys of the general top-k path][id list, list_cap
// entries and kWave trash slots]
size_t step_list_offset(int32_t out_blocks_max, int32_t n_slots_max) {
  return select_lds_bytes(out_blocks_max, n_slots_max) / sizeof(uint32_t);
}

template <typename TE, int D, int KIND, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_step(StepParams p, int list_off) {
  __shared__ StepShared<D, G> sh;
  extern __shared__ uint32_t dyn[];
  int32_t* list = reinterpret_cast<int32_t*>(dyn + list_off);
  const int NC = p.n_chunks, NS = p.dec.n_splits;
  const int n_score = p.units * NC;
  for (int t = blockIdx.x; t < p.total; t += gridDim.x) {
    if (t < n_score) {
      const int unit = t / NC;
      score_chunk<TE, D, KIND, G>(p.sel, unit, t % NC, sh.t);
      __builtin_amdgcn_s_waitcnt(0);  // this thread's published scores are stored
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(counter_of(p.sel.counters, unit), 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int unit = (t - n_score) / NS, split = (t - n_score) % NS;
      const UnitGeom ug = unit_geom(p.sel, unit);  // its loads overlap the wait
      if (threadIdx.x == 0) {
        const int32_t* cnt = counter_of(p.sel.counters, unit);
        const long long t0 = wall_clock64();
        for (int i = 0; published_i32(cnt) < NC; ++i) {
          __builtin_amdgcn_s_sleep(4);
          if ((i & 63) == 63 && wall_clock64() - t0 > p.wait_ticks) {
            publish_i32(p.ctrl + kCtrlStatus, HS_STEP_WAIT_EXPIRED);
            break;
          }
        }
      }
      __syncthreads();
      const bool writer = split == 0;
      const int cnt = select_from_scores(
          p.sel, unit, ug, sh.t, dyn, list,
          writer ? p.sel.out_ids + (int64_t)unit * p.sel.out_cap : nullptr,
          writer ? p.sel.out_cnt + unit : nullptr);
      int e0, e1;
      split_range(cnt, NS, split, e0, e1);
      decode_split<TE, D, G>(p.dec, unit, split, list, e0, e1, sh.d);
    }
    __syncthreads();  // LDS is reused by the next task
  }
}

// Workgroups of kernel k (256 threads, lds dynamic bytes) that the current
// device holds at once.
hipError_t resident_workgroups(const void* k, size_t lds, int* n) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, lds);
  if (e != hipSuccess) return e;
  *n = cus * per_cu;
  return *n > 0 ? hipSuccess : hipErrorInvalidConfiguration;
}

}  // namespace

// A quarter of a second of the device's wall clock (a scoring task takes
// microseconds).
hipError_t wait_bound(long long* ticks) {
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  *ticks = (long long)(khz > 0 ? khz : 100000) * 250;
  return hipSuccess;
}

namespace {

template <typename TE, int D, int KIND, int G>
hipError_t launch_one(StepParams p, size_t lds, int list_off, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&k_step<TE, D, KIND, G>);
  int r = 0;
  hipError_t e = resident_workgroups(k, lds, &r);
  if (e == hipSuccess) e = wait_bound(&p.wait_ticks);
  if (e != hipSuccess) return e;
  const dim3 grid(r < p.total ? r : p.total);
  hipLaunchKernelGGL((k_step<TE, D, KIND, G>), grid, dim3(256), lds, s, p, list_off);
  return hipGetLastError();
}

template <typename TE, int D, int KIND>
hipError_t launch_g(const StepParams& p, size_t lds, int list_off, hipStream_t s) {
  switch (p.sel.G) {
    case 1: return launch_one<TE, D, KIND, 1>(p, lds, list_off, s);
    case 2: return launch_one<TE, D, KIND, 2>(p, lds, list_off, s);
    case 4: return launch_one<TE, D, KIND, 4>(p, lds, list_off, s);
    default: return launch_one<TE, D, KIND, 8>(p, lds, list_off, s);
  }
}

template <typename TE, int D>
hipError_t launch_k(const StepParams& p, size_t lds, int list_off, hipStream_t s) {
  return p.sel.kind == HS_SUMMARY_MEAN ? launch_g<TE, D, HS_SUMMARY_MEAN>(p, lds, list_off, s)
                                       : launch_g<TE, D, HS_SUMMARY_MINMAX>(p, lds, list_off, s);
}

}  // namespace

int step_chunks(int32_t n_slots_max) { return select_chunks(n_slots_max); }

bool step_fits(int32_t out_blocks_max, int32_t n_slots_max, int32_t list_cap) {
  const size_t words = step_list_offset(out_blocks_max, n_slots_max) + (size_t)list_cap + kWave;
  return words * sizeof(uint32_t) <= kMaxDynLds;
}

hipError_t launch_step(const StepParams& p, hipStream_t s) {
  const int list_off = (int)step_list_offset(p.sel.out_blocks_max, p.sel.n_slots_max);
  const size_t lds = sizeof(uint32_t) * ((size_t)list_off + p.list_cap + kWave);
  const bool bf = p.sel.kv.elem_bytes == 2;
  if (p.sel.kv.head_dim == 64)
    return bf ? launch_k<bf16_t, 64>(p, lds, list_off, s) : launch_k<float, 64>(p, lds, list_off, s);
  return bf ? launch_k<bf16_t, 128>(p, lds, list_off, s) : launch_k<float, 128>(p, lds, list_off, s);
}

}  // namespace hs
