// Model extras (the nanochat walkthrough, "1. GPT model (nanochat/gpt.py)",
// efficiency tricks): per-layer residual mixing x <- lr x + l0 x0 (backout
// of a mid-layer residual is the case lr = 1, l0 = -lambda) and smear, a
// gated mix of the previous token's embedding, y_t = x_t + g_t x_(t-1),
// g_t = lambda sigmoid(w . x_t[:24]) (no mix at a row's first position).
// The scalars are device values of the storage type (parameters), their
// gradients fp32 device values reduced in a fixed order (per-block partials,
// then one block), written or added to.  The mix kernels also serve as the
// stream's plain add and its backout, and may work in place.  HBM-bound streams; smear takes one wave per token.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gk {

namespace {
constexpr int kMixBlocks = 1024;
constexpr int kSmearCh = 24;
constexpr int kSmearBlocks = 1024;

__device__ __forceinline__ float sigmoidf(float z) { return 1.f / (1.f + expf(-z)); }

template <typename T>
__device__ __forceinline__ void ld8(const T* p, int64_t i, float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = ld(p, i + e);
}
template <>
__device__ __forceinline__ void ld8<bf16>(const bf16* p, int64_t i, float* v) {
  const uint4 u = *(const uint4*)(p + i);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
template <typename T>
__device__ __forceinline__ void st8(T* p, int64_t i, const float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) st(p, i + e, v[e]);
}
template <>
__device__ __forceinline__ void st8<bf16>(bf16* p, int64_t i, const float* v) {
  uint4 u;
  u.x = pack2bf(v[0], v[1]);
  u.y = pack2bf(v[2], v[3]);
  u.z = pack2bf(v[4], v[5]);
  u.w = pack2bf(v[6], v[7]);
  *(uint4*)(p + i) = u;
}

__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}
}  // namespace

// the two weights of a mix: MIX_LAMBDAS (lam[0], lam[1]); MIX_BACKOUT (1,
// -lam[0]); MIX_ADD (1, 1), lam unused
template <typename T>
__device__ __forceinline__ void mix_weights(const T* lam, int mode, float& lr, float& l0) {
  lr = 1.f;
  l0 = 1.f;
  if (mode == MIX_LAMBDAS) {
    lr = ld(lam, 0);
    l0 = ld(lam, 1);
  } else if (mode == MIX_BACKOUT) {
    l0 = -ld(lam, 0);
  }
}

// y = lr x + l0 x0 (one rounding), runs of 8; y may be x (each thread reads
// its run before writing it)
template <typename T>
__global__ __launch_bounds__(256) void k_resid_mix_fwd(const T* x, const T* __restrict__ x0,
                                                       T* y, int64_t n8,
                                                       const T* __restrict__ lam, int mode) {
  float lr, l0;
  mix_weights(lam, mode, lr, l0);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    float a[8], b[8];
    ld8(x, 8 * i, a);
    ld8(x0, 8 * i, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = fmaf(lr, a[e], l0 * b[e]);
    st8(y, 8 * i, a);
  }
}

// dx = lr dy (dx may be dy); dx0 (+)= l0 dy; per-block partials of the
// scalars' gradients: MIX_LAMBDAS (sum dy x, sum dy x0); MIX_BACKOUT
// (-sum dy x0, unused), x not read
template <typename T>
__global__ __launch_bounds__(256) void k_resid_mix_bwd(
    const T* dy, const T* __restrict__ x, const T* __restrict__ x0, T* dx,
    T* __restrict__ dx0, int accumulate, int64_t n8, const T* __restrict__ lam, int mode,
    double* __restrict__ part) {
  __shared__ double red[4];
  float lr, l0;
  mix_weights(lam, mode, lr, l0);
  const bool want_x = mode == MIX_LAMBDAS;
  float sx = 0.f, s0 = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    float g[8], a[8], b[8], o[8];
    ld8(dy, 8 * i, g);
    if (want_x) ld8(x, 8 * i, a);
    ld8(x0, 8 * i, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (want_x) sx = fmaf(g[e], a[e], sx);
      s0 = fmaf(g[e], b[e], s0);
      o[e] = lr * g[e];
    }
    if (dx) st8(dx, 8 * i, o);
    if (accumulate) ld8(dx0, 8 * i, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = accumulate ? fmaf(l0, g[e], b[e]) : l0 * g[e];
    st8(dx0, 8 * i, o);
  }
  const double tx = block_sum_d(sx, red);
  const double t0 = block_sum_d(s0, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = want_x ? tx : -t0;
    part[2 * blockIdx.x + 1] = t0;
  }
}

// out[k] (fp32) = (out[k] if accumulate) + sum over `nparts` partial records
// spaced `stride` apart (k < width <= stride), fixed order: thread t sums
// records t, t + 256, ..., then a fixed shuffle tree and the four waves in
// order; one block
__global__ __launch_bounds__(256) void k_sum_parts(const double* __restrict__ part, int nparts,
                                                   int stride, int width, int accumulate,
                                                   float* __restrict__ out) {
  __shared__ double red[4];
  for (int k = 0; k < width; ++k) {
    double v = 0.0;
    for (int p = threadIdx.x; p < nparts; p += 256) v += part[(int64_t)p * stride + k];
    v = block_sum_d(v, red);
    if (threadIdx.x == 0) out[k] = accumulate ? out[k] + (float)v : (float)v;
  }
}

// smear forward: one wave per token n = b T + t
template <typename T>
__global__ __launch_bounds__(256) void k_smear_fwd(const T* __restrict__ x, int64_t rows,
                                                   int Tn, int D, const T* __restrict__ w,
                                                   const T* __restrict__ lam, T* __restrict__ y,
                                                   float* __restrict__ gate) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= rows) return;
  const T* xr = x + n * D;
  float z = lane < kSmearCh ? ld(xr, lane) * ld(w, lane) : 0.f;
  z = wave_sum(z);
  const bool first = n % Tn == 0;
  const float g = first ? 0.f : ld(lam, 0) * sigmoidf(z);
  if (lane == 0) gate[n] = g;
  const T* pr = xr - D;
  for (int c = 8 * lane; c < D; c += 512) {
    float a[8], b[8];
    ld8(xr, c, a);
    if (!first) {
      ld8(pr, c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = fmaf(g, b[e], a[e]);
    }
    st8(y + n * D, c, a);
  }
}

// smear backward: dx_t = dy_t + g_(t+1) dy_(t+1) (+ dz_t w on the first 24
// channels), dg_t = dy_t . x_(t-1), dz_t = dg_t lambda s (1 - s); per-block
// partials of dw (24) and dlambda
template <typename T>
__global__ __launch_bounds__(256) void k_smear_bwd(const T* __restrict__ dy,
                                                   const T* __restrict__ x, int64_t rows,
                                                   int Tn, int D, const T* __restrict__ w,
                                                   const T* __restrict__ lam,
                                                   const float* __restrict__ gate,
                                                   T* __restrict__ dx,
                                                   double* __restrict__ part) {
  __shared__ double red[4][kSmearCh + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float lm = ld(lam, 0);
  double accw = 0.0, accl = 0.0;     // lane < 24: dw[lane]; lane 24: dlambda
  for (int64_t n = (int64_t)blockIdx.x * 4 + wave; n < rows; n += (int64_t)gridDim.x * 4) {
    const bool first = n % Tn == 0, last = n % Tn == Tn - 1;
    const T* dyr = dy + n * D;
    const T* xr = x + n * D;
    float dg = 0.f;
    if (!first) {
      for (int c = 8 * lane; c < D; c += 512) {
        float a[8], b[8];
        ld8(dyr, c, a);
        ld8(xr - D, c, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) dg = fmaf(a[e], b[e], dg);
      }
      dg = wave_sum(dg);
    }
    const float xc = lane < kSmearCh ? ld(xr, lane) : 0.f;
    const float z = wave_sum(lane < kSmearCh ? xc * ld(w, lane) : 0.f);
    const float s = sigmoidf(z);
    const float dz = first ? 0.f : dg * lm * s * (1.f - s);
    const float gn = last ? 0.f : gate[n + 1];
    for (int c = 8 * lane; c < D; c += 512) {
      float a[8], b[8];
      ld8(dyr, c, a);
      if (!last) {
        ld8(dyr + D, c, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = fmaf(gn, b[e], a[e]);
      }
      if (c < kSmearCh) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < kSmearCh) a[e] = fmaf(dz, ld(w, c + e), a[e]);
      }
      st8(dx + n * D, c, a);
    }
    if (lane < kSmearCh) accw += (double)dz * xc;
    if (lane == kSmearCh && !first) accl += (double)dg * s;
  }
  if (lane <= kSmearCh) red[wave][lane] = lane < kSmearCh ? accw : accl;
  __syncthreads();
  if (threadIdx.x <= kSmearCh) {
    const double v = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                     (red[2][threadIdx.x] + red[3][threadIdx.x]);
    part[(int64_t)blockIdx.x * (kSmearCh + 1) + threadIdx.x] = v;
  }
}

// p[0..n) = 0 with 4-byte stores (any float alignment)
__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(1024, cdiv(n, 256)));
  GK_LAUNCH(Work(0.0, 4.0 * n), k_zero_f32, dim3(nb), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

size_t resid_mix_bwd_scratch_bytes() { return kMixBlocks * 2 * sizeof(double); }
size_t smear_bwd_scratch_bytes() { return kSmearBlocks * (kSmearCh + 1) * sizeof(double); }

hipError_t resid_mix_fwd(const void* x, const void* x0, void* y, int64_t n, const void* lam,
                         DType dt, hipStream_t s, int mode) {
  const int64_t n8 = n / 8;
  const unsigned nb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(4096, cdiv(n8, 256)));
  const Work w(0.0, 3.0 * n * (dt == BF16 ? 2 : 4));
  if (dt == BF16)
    GK_LAUNCH(w, k_resid_mix_fwd<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)x,
              (const bf16*)x0, (bf16*)y, n8, (const bf16*)lam, mode);
  else
    GK_LAUNCH(w, k_resid_mix_fwd<float>, dim3(nb), dim3(256), 0, s, (const float*)x,
              (const float*)x0, (float*)y, n8, (const float*)lam, mode);
  return hipGetLastError();
}

hipError_t resid_mix_bwd(const void* dy, const void* x, const void* x0, void* dx, void* dx0,
                         int accumulate, int64_t n, const void* lam, float* dlam, void* scratch,
                         DType dt, hipStream_t s, int mode, int accumulate_dlam) {
  const int64_t n8 = n / 8;
  const unsigned nb =
      (unsigned)std::max<int64_t>(1, std::min<int64_t>(kMixBlocks, cdiv(n8, 256 * 4)));
  double* part = (double*)scratch;
  const int es = dt == BF16 ? 2 : 4;
  const int reads = 2 + (mode == MIX_LAMBDAS ? 1 : 0) + (accumulate ? 1 : 0);
  const Work w(0.0, (double)n * es * (reads + (dx ? 1 : 0) + 1));
  if (dt == BF16)
    GK_LAUNCH(w, k_resid_mix_bwd<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)dy,
              (const bf16*)x, (const bf16*)x0, (bf16*)dx, (bf16*)dx0, accumulate, n8,
              (const bf16*)lam, mode, part);
  else
    GK_LAUNCH(w, k_resid_mix_bwd<float>, dim3(nb), dim3(256), 0, s, (const float*)dy,
              (const float*)x, (const float*)x0, (float*)dx, (float*)dx0, accumulate, n8,
              (const float*)lam, mode, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GK_LAUNCH(Work(), k_sum_parts, dim3(1), dim3(256), 0, s, (const double*)part, (int)nb, 2,
            mode == MIX_LAMBDAS ? 2 : 1, accumulate_dlam, dlam);
  return hipGetLastError();
}

hipError_t smear_fwd(const void* x, int64_t rows, int T, int D, const void* w, const void* lam,
                     void* y, float* gate, DType dt, hipStream_t s) {
  const unsigned nb = (unsigned)cdiv(rows, 4);
  const Work wk(0.0, (double)rows * D * (dt == BF16 ? 2 : 4) * 3 + 4.0 * rows);
  if (dt == BF16)
    GK_LAUNCH(wk, k_smear_fwd<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)x, rows, T, D,
              (const bf16*)w, (const bf16*)lam, (bf16*)y, gate);
  else
    GK_LAUNCH(wk, k_smear_fwd<float>, dim3(nb), dim3(256), 0, s, (const float*)x, rows, T, D,
              (const float*)w, (const float*)lam, (float*)y, gate);
  return hipGetLastError();
}

hipError_t smear_bwd(const void* dy, const void* x, int64_t rows, int T, int D, const void* w,
                     const void* lam, const float* gate, void* dx, float* dw_dlam,
                     void* scratch, DType dt, hipStream_t s, int accumulate_dw) {
  const unsigned nb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(kSmearBlocks,
                                                                         cdiv(rows, 16)));
  double* part = (double*)scratch;
  const Work wk(0.0, (double)rows * D * (dt == BF16 ? 2 : 4) * 4 + 4.0 * rows);
  if (dt == BF16)
    GK_LAUNCH(wk, k_smear_bwd<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)dy,
              (const bf16*)x, rows, T, D, (const bf16*)w, (const bf16*)lam, gate, (bf16*)dx,
              part);
  else
    GK_LAUNCH(wk, k_smear_bwd<float>, dim3(nb), dim3(256), 0, s, (const float*)dy,
              (const float*)x, rows, T, D, (const float*)w, (const float*)lam, gate, (float*)dx,
              part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dw[0..24) and dlambda at [24]
  GK_LAUNCH(Work(), k_sum_parts, dim3(1), dim3(256), 0, s, (const double*)part, (int)nb,
            kSmearCh + 1, kSmearCh + 1, accumulate_dw, dw_dlam);
  return hipGetLastError();
}

}  // namespace gk
