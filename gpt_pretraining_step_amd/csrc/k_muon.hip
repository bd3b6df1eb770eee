// Muon's orthogonalization of a matrix update (the nanochat walkthrough, "2.
// Muon optimizer": a quintic Newton-Schulz iteration, "Polar Express").
//
// Per tuple (a, b, c) the page's step is A = X^T X, B = b A + c A A,
// X <- a X + X B.  Here it runs as X <- X B' with B' = a I + b A + c A A
// (the same matrix, the identity term folded in), so each step is three
// products on the MFMA GEMM kernels plus two small elementwise passes over
// the s x s Gram matrix (s = the smaller side).  A matrix with fewer rows
// than columns is iterated in the transposed form of the same step: A =
// X X^T, X <- B' X.  X is bf16 between steps (A, B' too); the Gram
// products accumulate in fp32, split along the long side when that fills
// the chip.  The start divides G by its Frobenius norm (+ eps), reduced in
// a fixed order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gk {

namespace {
constexpr int kNormParts = 1024;
}

// per-block sum of squares (fp32 per thread, fp64 across the block)
template <typename T>
__global__ __launch_bounds__(256) void k_ns_sumsq(const T* __restrict__ g, int64_t n,
                                                  double* __restrict__ part) {
  __shared__ double red[4];
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    acc = fmaf(ld(g, i), ld(g, i), acc);
  double v = acc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// X = bf16(G / (||G|| + eps)); every block sums the partials in the same
// order
template <typename T>
__global__ __launch_bounds__(256) void k_ns_start(const T* __restrict__ g, int64_t n,
                                                  const double* __restrict__ part, int nparts,
                                                  float eps, bf16* __restrict__ x) {
  __shared__ double red[4];
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

__global__ __launch_bounds__(256) void k_ns_round(const float* __restrict__ a32, int64_t n,
                                                  bf16* __restrict__ a16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) a16[i] = f2bf(a32[i]);
}

// B' = bf16(a I + b A + c S), s x s
__global__ __launch_bounds__(256) void k_ns_combine(const bf16* __restrict__ A,
                                                    const float* __restrict__ S, int s, float a,
                                                    float b, float c, bf16* __restrict__ Bp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)s * s) return;
  const float diag = (i / s == i % s) ? a : 0.f;
  Bp[i] = f2bf(fmaf(c, S[i], fmaf(b, bf2f(A[i]), diag)));
}

namespace {
struct NsLayout {
  int64_t s, big;            // smaller and larger side
  size_t x, a32, a16, sq, bp, part, gscr, total;
};
size_t pad(size_t b) { return (b + 255) / 256 * 256; }
NsLayout ns_layout(int64_t m, int64_t n) {
  NsLayout L;
  L.s = std::min(m, n);
  L.big = std::max(m, n);
  size_t off = 0;
  L.x = off;    off += pad((size_t)m * n * 2);
  L.a32 = off;  off += pad((size_t)L.s * L.s * 4);
  L.a16 = off;  off += pad((size_t)L.s * L.s * 2);
  L.sq = off;   off += pad((size_t)L.s * L.s * 4);
  L.bp = off;   off += pad((size_t)L.s * L.s * 2);
  L.part = off; off += pad(kNormParts * sizeof(double));
  L.gscr = off;
  off += pad(std::max(gemm_scratch_bytes(L.s, L.s, L.big), gemm_scratch_bytes(L.s, L.s, L.s)));
  L.total = off;
  return L;
}
}  // namespace

size_t polar_express_ws_bytes(int64_t m, int64_t n) { return ns_layout(m, n).total; }

hipError_t polar_express(const void* g, int64_t m, int64_t n, DType dt, const float* coeffs,
                         int steps, float eps, void* x_out, void* ws, hipStream_t s) {
  const NsLayout L = ns_layout(m, n);
  char* w = (char*)ws;
  const int64_t mn = m * n, ss = L.s * L.s;
  double* part = (double*)(w + L.part);
  const int parts = (int)std::max<int64_t>(1, std::min<int64_t>(kNormParts, cdiv(mn, 2048)));
  const double gb = (double)mn * (dt == BF16 ? 2 : 4);
  // X_k lives in buf[k % 2]; the last one must be x_out
  bf16* buf[2];
  buf[steps % 2] = (bf16*)x_out;
  buf[(steps + 1) % 2] = (bf16*)(w + L.x);
  if (dt == BF16) {
    GK_LAUNCH(Work(0.0, gb), k_ns_sumsq<bf16>, dim3(parts), dim3(256), 0, s, (const bf16*)g, mn,
              part);
    GK_LAUNCH(Work(0.0, gb + 2.0 * mn), k_ns_start<bf16>, dim3(parts), dim3(256), 0, s,
              (const bf16*)g, mn, part, parts, eps, buf[0]);
  } else {
    GK_LAUNCH(Work(0.0, gb), k_ns_sumsq<float>, dim3(parts), dim3(256), 0, s, (const float*)g, mn,
              part);
    GK_LAUNCH(Work(0.0, gb + 2.0 * mn), k_ns_start<float>, dim3(parts), dim3(256), 0, s,
              (const float*)g, mn, part, parts, eps, buf[0]);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* a32 = (float*)(w + L.a32);
  bf16* a16 = (bf16*)(w + L.a16);
  float* sq = (float*)(w + L.sq);
  bf16* bp = (bf16*)(w + L.bp);
  void* gscr = w + L.gscr;
  const size_t gscr_bytes = L.total - L.gscr;
  const bool tall = m >= n;
  const unsigned eb = (unsigned)cdiv(ss, 256);
  for (int k = 0; k < steps; ++k) {
    const bf16* X = buf[k % 2];
    bf16* Xn = buf[(k + 1) % 2];
    // A = X^T X (tall: TN over the m rows) or X X^T (wide: NT over the n columns)
    GemmDesc ga = tall ? GemmDesc{OP_TN, L.s, L.s, m, X, n, X, n, a32, L.s, E_F32, nullptr,
                                  gscr, gscr_bytes}
                       : GemmDesc{OP_NT, L.s, L.s, n, X, n, X, n, a32, L.s, E_F32, nullptr,
                                  gscr, gscr_bytes};
    if ((e = gemm(ga, BF16, s)) != hipSuccess) return e;
    GK_LAUNCH(Work(0.0, 6.0 * ss), k_ns_round, dim3(eb), dim3(256), 0, s, a32, ss, a16);
    // S = A A
    GemmDesc gs{OP_NN, L.s, L.s, L.s, a16, L.s, a16, L.s, sq, L.s, E_F32, nullptr, gscr,
                gscr_bytes};
    if ((e = gemm(gs, BF16, s)) != hipSuccess) return e;
    GK_LAUNCH(Work(0.0, 8.0 * ss), k_ns_combine, dim3(eb), dim3(256), 0, s, a16, sq, (int)L.s,
              coeffs[3 * k], coeffs[3 * k + 1], coeffs[3 * k + 2], bp);
    // X <- X B' (tall) or B' X (wide)
    GemmDesc gx = tall ? GemmDesc{OP_NN, m, n, n, X, n, bp, n, Xn, n, E_STORE, nullptr,
                                  nullptr, 0}
                       : GemmDesc{OP_NN, m, n, m, bp, m, X, n, Xn, n, E_STORE, nullptr,
                                  nullptr, 0};
    if ((e = gemm(gx, BF16, s)) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gk
