// Fused GEMM epilogues: what happens to one fp32 accumulator at (m, n).
#pragma once
#include "common.h"
#include "kernels.h"

namespace gk {

template <typename Tv, int EPI>
__device__ __forceinline__ void epi_apply(void* Cv, void* auxv, int64_t ldc, int64_t m,
                                          int64_t n, float acc) {
  const int64_t i = m * ldc + n;
  if constexpr (EPI == E_STORE) {
    st((Tv*)Cv, i, acc);
  } else if constexpr (EPI == E_RESADD) {          // residual: C + acc, one rounding
    Tv* C = (Tv*)Cv;
    st(C, i, ld(C, i) + acc);
  } else if constexpr (EPI == E_RELU2) {           // a = relu(u)^2, u = acc rounded to Tv
    const float u = rnd_as((const Tv*)Cv, acc);
    const float r = fmaxf(u, 0.f);
    st((Tv*)Cv, i, r * r);
  } else if constexpr (EPI == E_DRELU2) {          // du = da * 2 relu(u), relu(u) = sqrt(a)
    const float a = ld((const Tv*)auxv, i);
    st((Tv*)Cv, i, acc * (2.0f * sqrtf(a)));
  } else if constexpr (EPI == E_F32) {
    ((float*)Cv)[i] = acc;
  } else {                                          // E_F32_ACC
    ((float*)Cv)[i] += acc;
  }
}

}  // namespace gk
