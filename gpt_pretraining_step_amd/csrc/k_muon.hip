// Muon's orthogonalization of a matrix update (the nanochat walkthrough, "2.
// Muon optimizer": a quintic Newton-Schulz iteration, "Polar Express").
//
// A step with coefficients (a, b, c) maps X to its odd quintic, a X +
// b X (X^T X) + c X (X^T X)^2, i.e. moves every singular value s to
// a s + b s^3 + c s^5 and keeps the singular vectors.  It is formed through
// the Gram matrix A = X^T X as X <- X P with P = a I + b A + c A A, so each
// step is three products on the MFMA GEMM kernels (A, A A, X P) plus one
// small elementwise pass over the s x s Gram matrix (s = the smaller
// side).  A matrix with fewer rows than columns takes the Gram matrix on
// the row side: A = X X^T, X <- P X.  X is bf16 between steps (A, B' too), products
// accumulate in fp32.  A batch of equally shaped matrices (the same
// parameter of every layer) runs in the same launches, one batch index per
// grid row, so the small products fill the chip.  The start divides G by
// its Frobenius norm (+ eps), reduced in a fixed order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gk {

namespace {
constexpr int kNormParts = 1024;
}

// per-block sum of squares (fp32 per thread, fp64 across the block); grid
// (parts, batch), matrix blockIdx.y of n elements
template <typename T>
__global__ __launch_bounds__(256) void k_ns_sumsq(const T* __restrict__ g, int64_t n,
                                                  double* __restrict__ part) {
  __shared__ double red[4];
  g += blockIdx.y * n;
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    acc = fmaf(ld(g, i), ld(g, i), acc);
  double v = acc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    part[blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// X = bf16(G / (||G|| + eps)) per matrix; every block sums its matrix's
// partials in the same order
template <typename T>
__global__ __launch_bounds__(256) void k_ns_start(const T* __restrict__ g, int64_t n,
                                                  const double* __restrict__ part, float eps,
                                                  bf16* __restrict__ x) {
  __shared__ double red[4];
  const int nparts = gridDim.x;
  part += blockIdx.y * nparts;
  g += blockIdx.y * n;
  x += blockIdx.y * n;
  double v = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) v += part[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double sum = (red[0] + red[1]) + (red[2] + red[3]);
  const float sc = (float)(1.0 / (sqrt(sum) + (double)eps));
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    x[i] = f2bf(ld(g, i) * sc);
}

// B' = bf16(a I + b A + c S) for every s x s matrix of the batch
__global__ __launch_bounds__(256) void k_ns_combine(const bf16* __restrict__ A,
                                                    const float* __restrict__ S, int s,
                                                    int64_t total, float a, float b, float c,
                                                    bf16* __restrict__ Bp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t e = i % ((int64_t)s * s);
  const float diag = (e / s == e % s) ? a : 0.f;
  Bp[i] = f2bf(fmaf(c, S[i], fmaf(b, bf2f(A[i]), diag)));
}

namespace {
struct NsLayout {
  int64_t s, big;            // smaller and larger side
  int parts;
  size_t x, a16, sq, bp, part, total;
};
size_t pad(size_t b) { return (b + 255) / 256 * 256; }
NsLayout ns_layout(int batch, int64_t m, int64_t n) {
  NsLayout L;
  L.s = std::min(m, n);
  L.big = std::max(m, n);
  L.parts = (int)std::max<int64_t>(1, std::min<int64_t>(kNormParts, cdiv(m * n, 4096)));
  const size_t ss = (size_t)batch * L.s * L.s;
  size_t off = 0;
  L.x = off;    off += pad((size_t)batch * m * n * 2);
  L.a16 = off;  off += pad(ss * 2);
  L.sq = off;   off += pad(ss * 4);
  L.bp = off;   off += pad(ss * 2);
  L.part = off; off += pad((size_t)batch * L.parts * sizeof(double));
  L.total = off;
  return L;
}
}  // namespace

size_t polar_express_ws_bytes(int batch, int64_t m, int64_t n) {
  return ns_layout(batch, m, n).total;
}

hipError_t polar_express(const void* g, int batch, int64_t m, int64_t n, DType dt,
                         const float* coeffs, int steps, float eps, void* x_out, void* ws,
                         hipStream_t s) {
  const NsLayout L = ns_layout(batch, m, n);
  char* w = (char*)ws;
  const int64_t mn = m * n, ss = L.s * L.s;
  double* part = (double*)(w + L.part);
  const double gb = (double)batch * mn * (dt == BF16 ? 2 : 4);
  // X_k lives in buf[k % 2]; the last one must be x_out
  bf16* buf[2];
  buf[steps % 2] = (bf16*)x_out;
  buf[(steps + 1) % 2] = (bf16*)(w + L.x);
  const dim3 ng(L.parts, batch);
  if (dt == BF16) {
    GK_LAUNCH(Work(0.0, gb), k_ns_sumsq<bf16>, ng, dim3(256), 0, s, (const bf16*)g, mn, part);
    GK_LAUNCH(Work(0.0, gb + 2.0 * batch * mn), k_ns_start<bf16>, ng, dim3(256), 0, s,
              (const bf16*)g, mn, part, eps, buf[0]);
  } else {
    GK_LAUNCH(Work(0.0, gb), k_ns_sumsq<float>, ng, dim3(256), 0, s, (const float*)g, mn, part);
    GK_LAUNCH(Work(0.0, gb + 2.0 * batch * mn), k_ns_start<float>, ng, dim3(256), 0, s,
              (const float*)g, mn, part, eps, buf[0]);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bf16* a16 = (bf16*)(w + L.a16);
  float* sq = (float*)(w + L.sq);
  bf16* bp = (bf16*)(w + L.bp);
  const bool tall = m >= n;
  const int64_t tot = (int64_t)batch * ss;
  const unsigned eb = (unsigned)cdiv(tot, 256);
  for (int k = 0; k < steps; ++k) {
    const bf16* X = buf[k % 2];
    bf16* Xn = buf[(k + 1) % 2];
    // A = X^T X (tall: TN over the m rows) or X X^T (wide: NT over the n
    // columns), rounded once to bf16
    const GemmDesc ga = tall ? GemmDesc{OP_TN, L.s, L.s, m, X, n, X, n, a16, L.s, E_STORE}
                             : GemmDesc{OP_NT, L.s, L.s, n, X, n, X, n, a16, L.s, E_STORE};
    if ((e = gemm_batched(ga, batch, mn, mn, ss, s)) != hipSuccess) return e;
    // S = A A (fp32)
    const GemmDesc gs{OP_NN, L.s, L.s, L.s, a16, L.s, a16, L.s, sq, L.s, E_F32};
    if ((e = gemm_batched(gs, batch, ss, ss, ss, s)) != hipSuccess) return e;
    GK_LAUNCH(Work(0.0, 8.0 * tot), k_ns_combine, dim3(eb), dim3(256), 0, s, a16, sq, (int)L.s,
              tot, coeffs[3 * k], coeffs[3 * k + 1], coeffs[3 * k + 2], bp);
    // X <- X B' (tall) or B' X (wide)
    const GemmDesc gx = tall ? GemmDesc{OP_NN, m, n, n, X, n, bp, n, Xn, n, E_STORE}
                             : GemmDesc{OP_NN, m, n, m, bp, m, X, n, Xn, n, E_STORE};
    if ((e = gemm_batched(gx, batch, tall ? mn : ss, tall ? ss : mn, mn, s)) != hipSuccess)
      return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gk
