// Kernel launch with optional per-launch timing.
//
// Every kernel of the library is launched through GK_LAUNCH.  While launch
// recording is on (gpt_prof_start), each launch goes through
// hipExtLaunchKernel with a start and a stop HIP event that the runtime ties
// to the kernel's own dispatch on its stream (the kernel's execution
// interval), and the launch's algorithmic work (matmul flops, compulsory HBM
// bytes) is kept beside them, so a caller can read per-kernel durations of a
// real step without a profiler.  When recording is off the cost is one load
// and branch per launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

// Algorithmic work of one launch: matmul flops and compulsory HBM bytes
// (0 where not stated).
struct Work {
  double flops, bytes;
  Work() : flops(0), bytes(0) {}
  Work(double f, double b) : flops(f), bytes(b) {}
};

extern volatile int g_prof_on;
// Reserves the next record for a launch of `kernel` on `s`: its two events,
// or false when the capacity is exhausted (the launch then goes unrecorded).
bool prof_slot(hipStream_t s, const void* kernel, Work w, hipEvent_t* start, hipEvent_t* stop);

// Visible (query, key) pairs of one head row of length T with window W:
// query i sees keys j with 0 <= i - j <= W.
inline double visible_pairs(int64_t T, int64_t W) {
  if (W > T - 1) W = T - 1;
  if (W < 0) return 0;
  return (double)(W + 1) * (W + 2) / 2 + (double)(T - W - 1) * (W + 1);
}

}  // namespace gk

#define GK_LAUNCH(WORK, K, GRID, BLOCK, SHMEM, STREAM, ...)                                  \
  do {                                                                                        \
    hipEvent_t gk_ev0_, gk_ev1_;                                                              \
    if (::gk::g_prof_on != 0 &&                                                               \
        ::gk::prof_slot((STREAM), reinterpret_cast<const void*>(&K), (WORK), &gk_ev0_, &gk_ev1_)) \
      hipExtLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, gk_ev0_, gk_ev1_, 0u, __VA_ARGS__); \
    else                                                                                      \
      hipLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                         \
  } while (0)
