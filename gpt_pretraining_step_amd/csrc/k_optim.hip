// The elementwise parts of the optimizer step (the nanochat walkthrough, "2.
// Muon optimizer": Muon for the block matrices, AdamW for embeddings,
// lm_head and value embeddings).  Muon: momentum with the Nesterov
// look-ahead feeding the orthogonalization, then W <- W (1 - lr wd) - lr X,
// X optionally rescaled per output row by NorMuon (an Adam-style second
// moment per neuron, then the update's Frobenius norm restored); AdamW with
// bias correction.  fp32 master weights, optionally written back
// as the bf16 copy the step reads.  HBM-bound streams of 4-float vectors.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gk {

namespace {
__device__ __forceinline__ void store4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
  uint2 o;
  o.x = pack2bf(v.x, v.y);
  o.y = pack2bf(v.z, v.w);
  *(uint2*)p = o;
}
__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4(const bf16* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
}  // namespace

// M <- beta M + (1 - beta) G; U = (1 - beta) G + beta M (Nesterov) or M
template <typename TU>
__global__ __launch_bounds__(256) void k_muon_momentum(const float* __restrict__ g,
                                                       float* __restrict__ mom,
                                                       TU* __restrict__ u, int64_t n4, float beta,
                                                       int nesterov) {
  const float omb = 1.f - beta;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 gv = load4(g + 4 * i);
    float4 m = load4(mom + 4 * i);
    m.x = fmaf(beta, m.x, omb * gv.x);
    m.y = fmaf(beta, m.y, omb * gv.y);
    m.z = fmaf(beta, m.z, omb * gv.z);
    m.w = fmaf(beta, m.w, omb * gv.w);
    store4(mom + 4 * i, m);
    float4 o = m;
    if (nesterov) {
      o.x = fmaf(beta, m.x, omb * gv.x);
      o.y = fmaf(beta, m.y, omb * gv.y);
      o.z = fmaf(beta, m.z, omb * gv.z);
      o.w = fmaf(beta, m.w, omb * gv.w);
    }
    store4(u + 4 * i, o);
  }
}

// W <- W (1 - lr wd) - lr X; optional bf16 copy
__global__ __launch_bounds__(256) void k_muon_update(float* __restrict__ w,
                                                     const bf16* __restrict__ x, int64_t n4,
                                                     float lr, float decay,
                                                     bf16* __restrict__ w16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 v = load4(w + 4 * i);
    const float4 xv = load4(x + 4 * i);
    v.x = fmaf(-lr, xv.x, v.x * decay);
    v.y = fmaf(-lr, xv.y, v.y * decay);
    v.z = fmaf(-lr, xv.z, v.z * decay);
    v.w = fmaf(-lr, xv.w, v.w * decay);
    store4(w + 4 * i, v);
    if (w16) store4(w16 + 4 * i, v);
  }
}

// AdamW: m, v moments; bc1 = 1 - beta1^t, bc2 = 1 - beta2^t
__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ w, const float* __restrict__ g,
                                               float* __restrict__ m, float* __restrict__ v,
                                               int64_t n4, float lr, float b1, float b2,
                                               float eps, float decay, float bc1, float bc2,
                                               bf16* __restrict__ w16) {
  const float r1 = 1.f / bc1, r2 = 1.f / bc2;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 gv = load4(g + 4 * i);
    float4 mv = load4(m + 4 * i), vv = load4(v + 4 * i), wv = load4(w + 4 * i);
    float* mp = &mv.x;
    float* vp = &vv.x;
    float* wp = &wv.x;
    const float* gp = &gv.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mp[e] = fmaf(b1, mp[e], (1.f - b1) * gp[e]);
      vp[e] = fmaf(b2, vp[e], (1.f - b2) * gp[e] * gp[e]);
      const float den = sqrtf(vp[e] * r2) + eps;
      wp[e] = fmaf(-lr, (mp[e] * r1) / den, wp[e] * decay);
    }
    store4(m + 4 * i, mv);
    store4(v + 4 * i, vv);
    store4(w + 4 * i, wv);
    if (w16) store4(w16 + 4 * i, wv);
  }
}

// The same two steps over the equally shaped matrices of one parameter group
// (the same tensor of every layer) in one launch: blockIdx.y picks the
// matrix, whose master / gradient / momentum sit at element offset
// offs.off[y] of the flat layout and whose update u / orthogonalized x is
// slot y of a contiguous [layers, n] staging buffer.
template <typename TU>
__global__ __launch_bounds__(256) void k_muon_momentum_group(const float* __restrict__ g,
                                                             float* __restrict__ mom,
                                                             TU* __restrict__ u, LayerOffsets offs,
                                                             int64_t n4, float beta,
                                                             int nesterov) {
  const int64_t off = offs.off[blockIdx.y];
  g += off;
  mom += off;
  u += (int64_t)blockIdx.y * n4 * 4;
  const float omb = 1.f - beta;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 gv = load4(g + 4 * i);
    float4 m = load4(mom + 4 * i);
    m.x = fmaf(beta, m.x, omb * gv.x);
    m.y = fmaf(beta, m.y, omb * gv.y);
    m.z = fmaf(beta, m.z, omb * gv.z);
    m.w = fmaf(beta, m.w, omb * gv.w);
    store4(mom + 4 * i, m);
    float4 o = m;
    if (nesterov) {
      o.x = fmaf(beta, m.x, omb * gv.x);
      o.y = fmaf(beta, m.y, omb * gv.y);
      o.z = fmaf(beta, m.z, omb * gv.z);
      o.w = fmaf(beta, m.w, omb * gv.w);
    }
    store4(u + 4 * i, o);
  }
}

// NorMuon's per-neuron statistics of the orthogonalized updates of a group
// (matrix blockIdx.y, rows [blockIdx.x NM_ROWS, +NM_ROWS)): per row r the
// mean square of X's row (fp32), the second moment v[r] <- b2 v[r] + (1 - b2)
// mean, the row's step size 1 / sqrt(max(v[r], floor)) to step[], and the
// block's two sums (mean, mean step^2) in fp64, in row order, to part[].
// One wave per row at a time, 8 bf16 per lane per load.
static constexpr int NM_ROWS = 16;
static constexpr float kNormuonFloor = 1e-10f;

__global__ __launch_bounds__(256) void k_normuon_stats(const bf16* __restrict__ x,
                                                       float* __restrict__ v, LayerOffsets offs,
                                                       int64_t rows, int64_t cols, float b2,
                                                       float* __restrict__ step,
                                                       double* __restrict__ part) {
  __shared__ double red[4][2];
  const int y = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  x += (int64_t)y * rows * cols;
  v += offs.off[y];
  step += (int64_t)y * rows;
  double s1 = 0.0, s2 = 0.0;
  for (int k = 0; k < NM_ROWS / 4; ++k) {
    const int64_t r = (int64_t)blockIdx.x * NM_ROWS + wave * (NM_ROWS / 4) + k;
    if (r >= rows) break;
    const bf16* xr = x + r * cols;
    float acc = 0.f;
    for (int64_t c = 8 * lane; c < cols; c += 512) {
      const uint4 u = *(const uint4*)(xr + c);
      const uint32_t* w = (const uint32_t*)&u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
        acc = fmaf(a, a, fmaf(b, b, acc));
      }
    }
    const float mean = wave_sum(acc) / (float)cols;
    const float vn = fmaf(b2, v[r], (1.f - b2) * mean);
    const float st = 1.f / sqrtf(fmaxf(vn, kNormuonFloor));
    if (lane == 0) {
      v[r] = vn;
      step[r] = st;
    }
    s1 += (double)mean;
    s2 += (double)mean * (double)st * (double)st;
  }
  if (lane == 0) {
    red[wave][0] = s1;
    red[wave][1] = s2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* p = part + ((int64_t)y * gridDim.x + blockIdx.x) * 2;
    p[0] = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
    p[1] = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
  }
}

// W <- W (1 - lr wd) - lr X, X optionally scaled per row by NorMuon's
// step[r] * sqrt(S1) / max(sqrt(S2), floor), (S1, S2) the matrix's sums over
// its nparts statistics blocks (re-reduced by every block in a fixed order,
// so there is no device-wide wait and the result is deterministic).
template <bool NORM>
__global__ __launch_bounds__(256) void k_muon_update_group(float* __restrict__ w,
                                                           const bf16* __restrict__ x,
                                                           LayerOffsets offs, int64_t n4,
                                                           float lr, float decay,
                                                           bf16* __restrict__ w16,
                                                           const float* __restrict__ step,
                                                           const double* __restrict__ part,
                                                           int nparts, int64_t cols) {
  const int64_t off = offs.off[blockIdx.y];
  w += off;
  x += (int64_t)blockIdx.y * n4 * 4;
  if (w16) w16 += off;
  float ratio = 1.f;
  if constexpr (NORM) {
    __shared__ float sratio;
    if (threadIdx.x < 64) {
      const double* p = part + (int64_t)blockIdx.y * nparts * 2;
      double a = 0.0, b = 0.0;
      for (int i = threadIdx.x; i < nparts; i += 64) {
        a += p[2 * i];
        b += p[2 * i + 1];
      }
      a = wave_sum_d(a);
      b = wave_sum_d(b);
      if (threadIdx.x == 0)
        sratio = (float)(sqrt(a) / fmax(sqrt(b), (double)kNormuonFloor));
    }
    __syncthreads();
    ratio = sratio;
    step += (int64_t)blockIdx.y * (n4 * 4 / cols);
  }
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 v = load4(w + 4 * i);
    const float4 xv = load4(x + 4 * i);
    float l = lr;
    if constexpr (NORM) l = lr * (step[(uint32_t)(4 * i) / (uint32_t)cols] * ratio);
    v.x = fmaf(-l, xv.x, v.x * decay);
    v.y = fmaf(-l, xv.y, v.y * decay);
    v.z = fmaf(-l, xv.z, v.z * decay);
    v.w = fmaf(-l, xv.w, v.w * decay);
    store4(w + 4 * i, v);
    if (w16) store4(w16 + 4 * i, v);
  }
}

namespace {
unsigned blocks_for(int64_t n4) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(2048, cdiv(n4, 256)));
}
}

hipError_t muon_momentum(const float* g, float* mom, void* u, int64_t n, float beta, int nesterov,
                         DType u_dt, hipStream_t s) {
  const int64_t n4 = n / 4;
  const Work w(0.0, n * (4.0 + 8.0 + (u_dt == BF16 ? 2.0 : 4.0)));
  if (u_dt == BF16)
    GK_LAUNCH(w, k_muon_momentum<bf16>, dim3(blocks_for(n4)), dim3(256), 0, s, g, mom, (bf16*)u,
              n4, beta, nesterov);
  else
    GK_LAUNCH(w, k_muon_momentum<float>, dim3(blocks_for(n4)), dim3(256), 0, s, g, mom,
              (float*)u, n4, beta, nesterov);
  return hipGetLastError();
}

hipError_t muon_update(float* w, const void* x, int64_t n, float lr, float wd, void* w16,
                       hipStream_t s) {
  const int64_t n4 = n / 4;
  const Work wk(0.0, n * (8.0 + 2.0 + (w16 ? 2.0 : 0.0)));
  GK_LAUNCH(wk, k_muon_update, dim3(blocks_for(n4)), dim3(256), 0, s, w, (const bf16*)x, n4, lr,
            1.f - lr * wd, (bf16*)w16);
  return hipGetLastError();
}

// per matrix about 2048 / layers blocks, so a group fills the chip as one
// large stream does
static unsigned group_blocks(int64_t n4, int layers) {
  const int64_t want = std::max<int64_t>(1, 2048 / std::max(layers, 1));
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, cdiv(n4, 256)));
}

hipError_t muon_momentum_group(const float* g, float* mom, void* u, const LayerOffsets& offs,
                               int layers, int64_t n, float beta, int nesterov, DType u_dt,
                               hipStream_t s) {
  if (layers < 1 || layers > kMaxGroupLayers || n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const dim3 grid(group_blocks(n4, layers), (unsigned)layers);
  const Work w(0.0, (double)layers * n * (4.0 + 8.0 + (u_dt == BF16 ? 2.0 : 4.0)));
  if (u_dt == BF16)
    GK_LAUNCH(w, k_muon_momentum_group<bf16>, grid, dim3(256), 0, s, g, mom, (bf16*)u, offs, n4,
              beta, nesterov);
  else
    GK_LAUNCH(w, k_muon_momentum_group<float>, grid, dim3(256), 0, s, g, mom, (float*)u, offs,
              n4, beta, nesterov);
  return hipGetLastError();
}

hipError_t muon_update_group(float* w, const void* x, const LayerOffsets& offs, int layers,
                             int64_t n, float lr, float wd, void* w16, hipStream_t s) {
  if (layers < 1 || layers > kMaxGroupLayers || n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const dim3 grid(group_blocks(n4, layers), (unsigned)layers);
  const Work wk(0.0, (double)layers * n * (8.0 + 2.0 + (w16 ? 2.0 : 0.0)));
  GK_LAUNCH(wk, k_muon_update_group<false>, grid, dim3(256), 0, s, w, (const bf16*)x, offs, n4,
            lr, 1.f - lr * wd, (bf16*)w16, (const float*)nullptr, (const double*)nullptr, 0,
            (int64_t)1);
  return hipGetLastError();
}

size_t normuon_scratch_bytes(int layers, int64_t rows) {
  const int64_t nparts = cdiv(rows, NM_ROWS);
  return (size_t)(((int64_t)layers * rows * 4 + 255) / 256 * 256) +
         (size_t)layers * nparts * 16;
}

hipError_t normuon_update_group(float* w, const void* x, float* v, const LayerOffsets& offs,
                                int layers, int64_t rows, int64_t cols, float b2, float lr,
                                float wd, void* w16, void* scratch, hipStream_t s) {
  if (layers < 1 || layers > kMaxGroupLayers || cols % 8 || rows < 1 ||
      rows > 65535 * NM_ROWS || rows * cols >= (int64_t)1 << 31)
    return hipErrorInvalidValue;
  const int64_t n = rows * cols, n4 = n / 4;
  const int nparts = (int)cdiv(rows, NM_ROWS);
  float* step = (float*)scratch;
  double* part = (double*)((char*)scratch + ((int64_t)layers * rows * 4 + 255) / 256 * 256);
  // statistics: X read once (bf16), v read and written, step written
  const Work ws(0.0, (double)layers * (n * 2.0 + rows * 12.0));
  GK_LAUNCH(ws, k_normuon_stats, dim3((unsigned)nparts, (unsigned)layers), dim3(256), 0, s,
            (const bf16*)x, v, offs, rows, cols, b2, step, part);
  const dim3 grid(group_blocks(n4, layers), (unsigned)layers);
  const Work wk(0.0, (double)layers * (n * (8.0 + 2.0 + (w16 ? 2.0 : 0.0)) + rows * 4.0));
  GK_LAUNCH(wk, k_muon_update_group<true>, grid, dim3(256), 0, s, w, (const bf16*)x, offs, n4,
            lr, 1.f - lr * wd, (bf16*)w16, (const float*)step, (const double*)part, nparts,
            cols);
  return hipGetLastError();
}

hipError_t adamw(float* w, const float* g, float* m, float* v, int64_t n, int step, float lr,
                 float b1, float b2, float eps, float wd, void* w16, hipStream_t s) {
  const int64_t n4 = n / 4;
  const float bc1 = (float)(1.0 - pow((double)b1, step));
  const float bc2 = (float)(1.0 - pow((double)b2, step));
  const Work wk(0.0, n * (4.0 + 3 * 8.0 + (w16 ? 2.0 : 0.0)));
  GK_LAUNCH(wk, k_adamw, dim3(blocks_for(n4)), dim3(256), 0, s, w, g, m, v, n4, lr, b1, b2, eps,
            1.f - lr * wd, bc1, bc2, (bf16*)w16);
  return hipGetLastError();
}

}  // namespace gk
