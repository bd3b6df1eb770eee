// GEMMs of the GPT step on gfx950.
//
//   NT  C[M,N] = A[M,K] B[N,K]^T    forward projections, y = x W^T
//   NN  C[M,N] = A[M,K] B[K,N]      input gradients,      dx = dy W
//   TN  C[M,N] = A[K,M]^T B[K,N]    weight gradients,     dW = dy^T x
//
// Every product accumulates in fp32 and finishes in a fused epilogue (plain
// store, residual add, ReLU^2, ReLU^2 backward, fp32 store / accumulate).
// The bf16 path runs on the MFMA kernel (gemm_mfma.h); the generic tiled
// kernel below covers fp32 storage and shapes the MFMA kernel does not take.
#include "common.h"
#include "gemm_epi.h"
#include "gemm_mfma.h"
#include "kernels.h"

namespace gk {

// Generic 64x64 tile, 16-deep K slices through LDS, 4x4 outputs per thread.
template <typename Tv, int OP, int EPI>
__global__ __launch_bounds__(256) void k_gemm_simple(int64_t M, int64_t N, int64_t K,
                                                     const Tv* A, int64_t lda, const Tv* B,
                                                     int64_t ldb, void* C, int64_t ldc,
                                                     void* aux) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      int ml, kl;
      if (OP == OP_TN) { ml = e & 63; kl = e >> 6; } else { kl = e & 15; ml = e >> 4; }
      int64_t m = m0 + ml, k = k0 + kl;
      float v = 0.f;
      if (m < M && k < K) v = (OP == OP_TN) ? ld(A, k * lda + m) : ld(A, m * lda + k);
      As[kl][ml] = v;
      int nl;
      if (OP == OP_NT) { kl = e & 15; nl = e >> 4; } else { nl = e & 63; kl = e >> 6; }
      int64_t n = n0 + nl;
      k = k0 + kl;
      v = 0.f;
      if (n < N && k < K) v = (OP == OP_NT) ? ld(B, n * ldb + k) : ld(B, k * ldb + n);
      Bs[kl][nl] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty + 16 * i]; b[i] = Bs[kk][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) epi_apply<Tv, EPI>(C, aux, ldc, m, n, acc[i][j]);
    }
}

template <typename Tv, int OP>
static hipError_t launch_simple_op(const GemmDesc& g, hipStream_t s) {
  dim3 grid((unsigned)cdiv(g.N, 64), (unsigned)cdiv(g.M, 64)), block(256);
  const Tv* A = (const Tv*)g.A;
  const Tv* B = (const Tv*)g.B;
  switch (g.epi) {
    case E_STORE:   GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_STORE>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    case E_RESADD:  GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_RESADD>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    case E_RELU2:   GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_RELU2>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    case E_DRELU2:  GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_DRELU2>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    case E_F32:     GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_F32>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    case E_F32_ACC: GK_LAUNCH(Work(), (k_gemm_simple<Tv, OP, E_F32_ACC>), grid, block, 0, s, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.C, g.ldc, g.aux); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename Tv>
static hipError_t launch_simple(const GemmDesc& g, hipStream_t s) {
  switch (g.op) {
    case OP_NT: return launch_simple_op<Tv, OP_NT>(g, s);
    case OP_NN: return launch_simple_op<Tv, OP_NN>(g, s);
    case OP_TN: return launch_simple_op<Tv, OP_TN>(g, s);
  }
  return hipErrorInvalidValue;
}

size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  return mfma_splitk_bytes(M, N, K);
}

hipError_t gemm(const GemmDesc& g, DType dt, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0) return hipErrorInvalidValue;
  if (dt == BF16) {
    if (mfma_gemm_supported(g)) return mfma_gemm(g, s);
    return launch_simple<bf16>(g, s);
  }
  return launch_simple<float>(g, s);
}

}  // namespace gk
