// Kernel launch with optional per-launch timing.
//
// Every kernel of the library is launched through GK_LAUNCH.  While launch
// recording is on (gpt_prof_start), each launch is bracketed by two HIP
// events recorded on the launch's own stream, and the launch's algorithmic
// work (matmul flops, compulsory HBM bytes) is kept beside them, so a caller
// can read per-kernel durations of a real step without a profiler.  When
// recording is off the cost is one load and branch per launch.
#pragma once
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
void prof_begin(hipStream_t s, const void* kernel, Work w);
void prof_end(hipStream_t s);

// Visible (query, key) pairs of one head row of length T with window W:
// query i sees keys j with 0 <= i - j <= W.
inline double visible_pairs(int64_t T, int64_t W) {
  if (W > T - 1) W = T - 1;
  if (W < 0) return 0;
  return (double)(W + 1) * (W + 2) / 2 + (double)(T - W - 1) * (W + 1);
}

}  // namespace gk

#define GK_LAUNCH(WORK, K, GRID, BLOCK, SHMEM, STREAM, ...)                       \
  do {                                                                             \
    const bool gk_rec_ = ::gk::g_prof_on != 0;                                     \
    if (gk_rec_) ::gk::prof_begin((STREAM), reinterpret_cast<const void*>(&K), (WORK)); \
    hipLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                \
    if (gk_rec_) ::gk::prof_end((STREAM));                                         \
  } while (0)
