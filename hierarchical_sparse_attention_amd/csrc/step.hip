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
// each launch pays its own ramp-up and drain. Here the units run as a
// dataflow inside one grid, so one unit's top-k or merge overlaps other
// units' HBM streams.
//
// Scheduling: a persistent grid of R workgroups, R = what the GPU holds at
// once (occupancy x compute units, from the HIP occupancy query), so every
// workgroup of the grid is resident together. Task t of the step goes to
// workgroup t % R, which runs its tasks in increasing t. Tasks are laid out
// in rounds: round r holds the scoring tasks of unit r (r < U), then the
// split tasks of unit r - L (r >= L), with lookahead L in [1, U], so every
// scoring task of a unit comes before all of its split tasks. The unit's
// last scoring task runs the top-k and raises the unit's ready flag; a split
// task waits for that flag before it reads the ids. Progress: take the
// waiting split task with the smallest t; the scoring tasks it waits for
// have smaller t, and each is either done or being run by its (resident)
// workgroup, whose current task has an even smaller t, so it waits for
// nothing and finishes. There is no shared ticket counter: device-scope
// atomics on one address serialise (about 12 ns each on MI355X), which for
// a thousand workgroups costs more than the fusion saves. The wait is still
// bounded (kMaxSpins polls): if the flag never comes, the task goes on with
// whatever ids are in memory (they are range-checked, so every access stays
// in bounds) and the kernel ends. The last split task of each unit clears
// the unit's flag, so flags are back at zero after the launch.
#include "decode_impl.h"
#include "select_impl.h"

namespace hs {
namespace {

constexpr int kMaxSpins = 1 << 21;  // polls of a ready flag (each at least a round trip)

struct Task {
  int unit, index;
  bool score;
};

__device__ __forceinline__ Task task_of(const StepParams& p, int t) {
  const int U = p.units, L = p.lookahead, NC = p.n_chunks, NS = p.n_splits;
  Task k;
  const int a = L * NC;  // rounds [0, L): scoring only
  if (t < a) {
    k.unit = t / NC;
    k.index = t % NC;
    k.score = true;
    return k;
  }
  t -= a;
  const int per = NC + NS;
  const int b = (U - L) * per;  // rounds [L, U): scoring of r, splits of r - L
  if (t < b) {
    const int r = L + t / per, i = t % per;
    k.score = i < NC;
    k.unit = k.score ? r : r - L;
    k.index = k.score ? i : i - NC;
    return k;
  }
  t -= b;  // rounds [U, U + L): splits of U - L ...
  k.unit = U - L + t / NS;
  k.index = t % NS;
  k.score = false;
  return k;
}

template <int D, int G>
union StepShared {
  TopkShared t;
  DecodeShared<D, G> d;
};

template <typename TE, int D, int KIND, int G>
__global__ __launch_bounds__(256) void k_step(StepParams p) {
  __shared__ StepShared<D, G> sh;
  extern __shared__ uint32_t dyn[];
  for (int t = blockIdx.x; t < p.total; t += gridDim.x) {
    const Task task = task_of(p, t);
    if (task.score) {
      if (select_task<TE, D, KIND, G>(p.sel, task.unit, task.index, p.n_chunks, sh.t, dyn)) {
        __builtin_amdgcn_s_waitcnt(0);  // ids and count are stored
        __syncthreads();
        if (threadIdx.x == 0) publish_i32(&p.ready[task.unit], 1);
      }
    } else {
      if (threadIdx.x == 0) {
        for (int i = 0; i < kMaxSpins && published_i32(&p.ready[task.unit]) == 0; ++i)
          __builtin_amdgcn_s_sleep(2);
      }
      __syncthreads();
      if constexpr (sizeof(TE) == 2)
        decode_task_bf16<D, G>(p.dec, task.unit, task.index, p.n_splits, sh.d);
      else
        decode_task_f32<D, G, f32_unroll<G>()>(p.dec, task.unit, task.index, p.n_splits, sh.d);
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

template <typename TE, int D, int KIND, int G>
hipError_t launch_one(const StepParams& p, size_t lds, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&k_step<TE, D, KIND, G>);
  int r = 0;
  const hipError_t e = resident_workgroups(k, lds, &r);
  if (e != hipSuccess) return e;
  const dim3 grid(r < p.total ? r : p.total);
  hipLaunchKernelGGL((k_step<TE, D, KIND, G>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

template <typename TE, int D, int KIND>
hipError_t launch_g(const StepParams& p, size_t lds, hipStream_t s) {
  switch (p.sel.G) {
    case 1: return launch_one<TE, D, KIND, 1>(p, lds, s);
    case 2: return launch_one<TE, D, KIND, 2>(p, lds, s);
    case 4: return launch_one<TE, D, KIND, 4>(p, lds, s);
    default: return launch_one<TE, D, KIND, 8>(p, lds, s);
  }
}

template <typename TE, int D>
hipError_t launch_k(const StepParams& p, size_t lds, hipStream_t s) {
  return p.sel.kind == HS_SUMMARY_MEAN ? launch_g<TE, D, HS_SUMMARY_MEAN>(p, lds, s)
                                       : launch_g<TE, D, HS_SUMMARY_MINMAX>(p, lds, s);
}

}  // namespace

int step_chunks(int32_t n_slots_max) { return select_chunks(n_slots_max); }

hipError_t launch_step(const StepParams& p, hipStream_t s) {
  const size_t lds = select_lds_bytes(p.sel.out_blocks_max, p.sel.n_slots_max);
  const bool bf = p.sel.kv.elem_bytes == 2;
  if (p.sel.kv.head_dim == 64)
    return bf ? launch_k<bf16_t, 64>(p, lds, s) : launch_k<float, 64>(p, lds, s);
  return bf ? launch_k<bf16_t, 128>(p, lds, s) : launch_k<float, 128>(p, lds, s);
}

}  // namespace hs
