// Token-id range check: the number of ids outside [0, V) in a token buffer,
// written to one int (no atomics, no prior zeroing: one workgroup walks the
// whole buffer and reduces in a fixed order).  Run ahead of the gathers when
// the caller asks for the check, so an out-of-range id is reported as an
// argument error instead of being used as a row index.
#include "common.h"
#include "kernels.h"

namespace gk {

__global__ __launch_bounds__(1024) void k_count_bad_ids(const int32_t* __restrict__ tok,
                                                        int64_t n, int V,
                                                        int* __restrict__ count) {
  __shared__ int red[16];
  int c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) c += (unsigned)tok[i] >= (unsigned)V;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < 16; ++w) t += red[w];
    *count = t;
  }
}

hipError_t count_bad_ids(const int32_t* tok, int64_t n, int V, int* count, hipStream_t s) {
  const Work w(0.0, n * 4.0 + 4.0);
  GK_LAUNCH(w, k_count_bad_ids, dim3(1), dim3(1024), 0, s, tok, n, V, count);
  return hipGetLastError();
}

}  // namespace gk
