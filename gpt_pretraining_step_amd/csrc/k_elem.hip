// HBM-bound kernels of the GPT step for gfx950: RMSNorm, rotary + QK-norm,
// token / value embeddings, cross-entropy and the loss / bits-per-byte
// reductions.  One 64-lane wavefront owns a row wherever a row reduction is
// needed, so reductions are register shuffles with no LDS round trip.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {

static constexpr int kBlock = 256;   // 4 wavefronts

// ------------------------------------------------------------------ utils
__global__ void k_fill_zero(uint4* p, int64_t n16, uint8_t* tail, int ntail) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// Zero-fill through a kernel (not a memset node), so a captured graph that
// replays it stays correct.
hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  int64_t n16 = bytes / 16;
  int ntail = (int)(bytes - n16 * 16);
  int64_t blocks = n16 ? cdiv(n16, kBlock) : 1;
  if (blocks > 4096) blocks = 4096;
  GK_LAUNCH(Work(), k_fill_zero, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                     (uint4*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  return hipGetLastError();
}

// ------------------------------------------------------------- transpose
// out[c, r] = in[r, c] for a [rows, cols] bf16 matrix (rows, cols multiples
// of 8): 64 x 64 tiles through LDS, 16-byte loads and stores.  grid
// (cdiv(cols, 64), cdiv(rows, 64)), 512 threads: thread t moves 8 values.
__global__ __launch_bounds__(512) void k_transpose16(const bf16* __restrict__ in, int64_t rows,
                                                     int64_t cols, bf16* __restrict__ out) {
  __shared__ bf16 tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tr = threadIdx.x >> 3, tc = 8 * (threadIdx.x & 7);
  if (r0 + tr < rows && c0 + tc < cols) {
    const uint4 v = *(const uint4*)(in + (r0 + tr) * cols + c0 + tc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[tc + e][tr] = (bf16)(w[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  // thread t writes out row c0 + t / 8, columns (= in rows) r0 + 8 (t % 8) ..
  const int64_t oc = c0 + tr, orr = r0 + tc;
  if (oc < cols && orr < rows) {
    uint4 o;
    uint32_t* ow = (uint32_t*)&o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = (uint32_t)tile[tr][tc + 2 * e] | ((uint32_t)tile[tr][tc + 2 * e + 1] << 16);
    *(uint4*)(out + oc * rows + orr) = o;
  }
}

hipError_t transpose_bf16(const void* in, int64_t rows, int64_t cols, void* out, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows, 64));
  GK_LAUNCH(Work(0.0, 4.0 * rows * cols), k_transpose16, grid, dim3(512), 0, s, (const bf16*)in,
            rows, cols, (bf16*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------- rope table
// (cos, sin) of theta_{t,j} = t * base^(-2j/hd), in double precision.
__global__ void k_rope_table(float2* cs, int T, int hd, double base) {
  int half = hd >> 1;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * half) return;
  int t = (int)(i / half), j = (int)(i % half);
  double a = (double)t * pow(base, -2.0 * (double)j / (double)hd);
  cs[i] = make_float2((float)cos(a), (float)sin(a));
}

hipError_t rope_table(float* cs, int T, int hd, float base, hipStream_t s) {
  int64_t n = (int64_t)T * (hd / 2);
  GK_LAUNCH(Work(), k_rope_table, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock),
                     0, s, (float2*)cs, T, hd, (double)base);
  return hipGetLastError();
}

// -------------------------------------------------------------- embedding
// Row copy in 16-byte units (row bytes a multiple of 16) or elements.
__global__ void k_embed_fwd16(const int32_t* tok, int T, const uint4* wte,
                              uint4* x, int units, int64_t total) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  int64_t n = i / units;
  int u = (int)(i % units);
  int id = tok[(n / T) * (T + 1) + n % T];
  x[i] = wte[(int64_t)id * units + u];
}
template <typename E>
__global__ void k_embed_fwd_el(const int32_t* tok, int T, const E* wte, E* x,
                               int D, int64_t total) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  int64_t n = i / D;
  int d = (int)(i % D);
  int id = tok[(n / T) * (T + 1) + n % T];
  x[i] = wte[(int64_t)id * D + d];
}

hipError_t embed_fwd(const int32_t* tok, int B, int T, const void* wte,
                     void* x, int D, DType dt, hipStream_t s) {
  int es = dt == BF16 ? 2 : 4;
  int64_t N = (int64_t)B * T;
  if (((int64_t)D * es) % 16 == 0) {
    int units = D * es / 16;
    int64_t total = N * units;
    GK_LAUNCH(Work(), k_embed_fwd16, dim3((unsigned)cdiv(total, kBlock)), dim3(kBlock),
                       0, s, tok, T, (const uint4*)wte, (uint4*)x, units, total);
  } else if (dt == BF16) {
    GK_LAUNCH(Work(), k_embed_fwd_el<uint16_t>, dim3((unsigned)cdiv(N * D, kBlock)),
                       dim3(kBlock), 0, s, tok, T, (const uint16_t*)wte, (uint16_t*)x, D, N * D);
  } else {
    GK_LAUNCH(Work(), k_embed_fwd_el<float>, dim3((unsigned)cdiv(N * D, kBlock)),
                       dim3(kBlock), 0, s, tok, T, (const float*)wte, (float*)x, D, N * D);
  }
  return hipGetLastError();
}

template <typename Tv>
__global__ void k_embed_bwd(const int32_t* tok, int T, const Tv* dx, int ldx,
                            float* dW, int D, int64_t total) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  int64_t n = i / D;
  int d = (int)(i % D);
  int id = tok[(n / T) * (T + 1) + n % T];
  atomicAdd(dW + (int64_t)id * D + d, ld(dx, n * ldx + d));
}

hipError_t embed_bwd(const int32_t* tok, int B, int T, const void* dx, int ldx,
                     float* dW, int D, DType dt, hipStream_t s) {
  int64_t total = (int64_t)B * T * D;
  if (dt == BF16)
    GK_LAUNCH(Work(), k_embed_bwd<bf16>, dim3((unsigned)cdiv(total, kBlock)), dim3(kBlock),
                       0, s, tok, T, (const bf16*)dx, ldx, dW, D, total);
  else
    GK_LAUNCH(Work(), k_embed_bwd<float>, dim3((unsigned)cdiv(total, kBlock)), dim3(kBlock),
                       0, s, tok, T, (const float*)dx, ldx, dW, D, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm
// One wavefront per row.  r = 1/sqrt(mean(x^2) + eps), y = x r.
template <typename Tv>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const Tv* x, Tv* y, float* r,
                                                     int64_t rows, int D, float eps) {
  int lane = threadIdx.x & 63;
  int64_t row = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const Tv* xr = x + row * D;
  float ss = 0.f;
  for (int d = lane; d < D; d += 64) {
    float v = ld(xr, d);
    ss += v * v;
  }
  ss = wave_sum(ss);
  float rr = 1.0f / sqrtf(ss / (float)D + eps);
  Tv* yr = y + row * D;
  for (int d = lane; d < D; d += 64) st(yr, d, ld(xr, d) * rr);
  if (lane == 0) r[row] = rr;
}

// bf16 rows with D % 8 == 0: 16-byte vectors, the row kept in registers.
// MIX: the row is first mixed, x = bf16(lam[0] x + lam[1] x0) (the model
// extras' residual mixing ahead of a block), stored to xout (may be x) and
// normalised as rounded.
template <int VPL, bool MIX = false>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_v(const bf16* x, bf16* y, float* r,
                                                       int64_t rows, int D, float eps,
                                                       const bf16* x0, const bf16* lam,
                                                       bf16* xout) {
  int lane = threadIdx.x & 63;
  int64_t row = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* xr = (const uint4*)(x + row * D);
  int nv = D >> 3;
  uint4 buf[VPL];
  float ss = 0.f;
  float lr = 0.f, l0 = 0.f;
  if constexpr (MIX) {
    lr = ld(lam, 0);
    l0 = ld(lam, 1);
  }
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    int v = lane + 64 * k;
    buf[k] = v < nv ? xr[v] : make_uint4(0, 0, 0, 0);
    if constexpr (MIX) {
      if (v < nv) {
        const uint4 u0 = ((const uint4*)(x0 + row * D))[v];
        uint32_t* w = (uint32_t*)&buf[k];
        const uint32_t* w0 = (const uint32_t*)&u0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack2bf(fmaf(lr, __uint_as_float(w[e] << 16), l0 * __uint_as_float(w0[e] << 16)),
                         fmaf(lr, __uint_as_float(w[e] & 0xFFFF0000u),
                              l0 * __uint_as_float(w0[e] & 0xFFFF0000u)));
        ((uint4*)(xout + row * D))[v] = buf[k];
      }
    }
    const uint32_t* w = (const uint32_t*)&buf[k];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
      ss += a * a + b * b;
    }
  }
  ss = wave_sum(ss);
  float rr = 1.0f / sqrtf(ss / (float)D + eps);
  uint4* yr = (uint4*)(y + row * D);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    int v = lane + 64 * k;
    if (v < nv) {
      const uint32_t* w = (const uint32_t*)&buf[k];
      uint4 o;
      uint32_t* ow = (uint32_t*)&o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ow[e] = pack2bf(__uint_as_float(w[e] << 16) * rr,
                        __uint_as_float(w[e] & 0xFFFF0000u) * rr);
      yr[v] = o;
    }
  }
  if (lane == 0) r[row] = rr;
}

hipError_t rmsnorm_fwd(const void* x, void* y, float* r, int64_t rows, int D,
                       float eps, DType dt, hipStream_t s) {
  dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  const Work w(0.0, (double)rows * D * 2 * (dt == BF16 ? 2 : 4) + rows * 4.0);  // x in, y out, r
  if (dt == BF16 && D % 8 == 0 && D <= 64 * 8 * 4) {
    int vpl = (int)cdiv(D / 8, 64);
    if (vpl == 1)
      GK_LAUNCH(w, k_rmsnorm_fwd_v<1>, grid, block, 0, s, (const bf16*)x, (bf16*)y, r, rows, D, eps,
                nullptr, nullptr, nullptr);
    else if (vpl == 2)
      GK_LAUNCH(w, k_rmsnorm_fwd_v<2>, grid, block, 0, s, (const bf16*)x, (bf16*)y, r, rows, D, eps,
                nullptr, nullptr, nullptr);
    else if (vpl == 3)
      GK_LAUNCH(w, k_rmsnorm_fwd_v<3>, grid, block, 0, s, (const bf16*)x, (bf16*)y, r, rows, D, eps,
                nullptr, nullptr, nullptr);
    else
      GK_LAUNCH(w, k_rmsnorm_fwd_v<4>, grid, block, 0, s, (const bf16*)x, (bf16*)y, r, rows, D, eps,
                nullptr, nullptr, nullptr);
  } else if (dt == BF16) {
    GK_LAUNCH(w, k_rmsnorm_fwd<bf16>, grid, block, 0, s, (const bf16*)x, (bf16*)y, r, rows, D, eps);
  } else {
    GK_LAUNCH(w, k_rmsnorm_fwd<float>, grid, block, 0, s, (const float*)x, (float*)y, r, rows, D, eps);
  }
  return hipGetLastError();
}

bool rmsnorm_fwd_mix_ok(int D, DType dt) { return dt == BF16 && D % 8 == 0 && D <= 64 * 8 * 4; }

hipError_t rmsnorm_fwd_mix(const void* x, const void* x0, const void* lam, void* xout, void* y,
                           float* r, int64_t rows, int D, float eps, DType dt, hipStream_t s) {
  if (!rmsnorm_fwd_mix_ok(D, dt)) return hipErrorInvalidValue;
  dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  const Work w(0.0, (double)rows * D * 2 * 4 + rows * 4.0);   // x, x0 in; xout, y out; r
  const int vpl = (int)cdiv(D / 8, 64);
#define GK_MIX_ARGS (const bf16*)x, (bf16*)y, r, rows, D, eps, (const bf16*)x0, (const bf16*)lam, \
                    (bf16*)xout
  if (vpl == 1)
    GK_LAUNCH(w, (k_rmsnorm_fwd_v<1, true>), grid, block, 0, s, GK_MIX_ARGS);
  else if (vpl == 2)
    GK_LAUNCH(w, (k_rmsnorm_fwd_v<2, true>), grid, block, 0, s, GK_MIX_ARGS);
  else if (vpl == 3)
    GK_LAUNCH(w, (k_rmsnorm_fwd_v<3, true>), grid, block, 0, s, GK_MIX_ARGS);
  else
    GK_LAUNCH(w, (k_rmsnorm_fwd_v<4, true>), grid, block, 0, s, GK_MIX_ARGS);
#undef GK_MIX_ARGS
  return hipGetLastError();
}

// dx = dres + r (g - y mean(g y)); g = dy plus, on the first C columns, the
// value-embedding gate term sum_kv vez[row, kv] wg[kv, c].
template <typename Tv>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const Tv* dy, const Tv* y, const float* r,
                                                     const Tv* dres, Tv* dx, int64_t rows, int D,
                                                     const float* vez, const Tv* wg, int Hkv, int C) {
  int lane = threadIdx.x & 63;
  int64_t row = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const Tv* dyr = dy + row * D;
  const Tv* yr = y + row * D;
  const float* vz = vez ? vez + row * Hkv : nullptr;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) {
    float g = ld(dyr, d);
    if (vz && d < C)
      for (int kv = 0; kv < Hkv; ++kv) g += vz[kv] * ld(wg, (int64_t)kv * C + d);
    acc += g * ld(yr, d);
  }
  float m = wave_sum(acc) / (float)D;
  float rr = r[row];
  for (int d = lane; d < D; d += 64) {
    float g = ld(dyr, d);
    if (vz && d < C)
      for (int kv = 0; kv < Hkv; ++kv) g += vz[kv] * ld(wg, (int64_t)kv * C + d);
    float v = rr * (g - ld(yr, d) * m);
    if (dres) v += ld(dres, row * D + d);
    st(dx, row * D + d, v);
  }
}

// bf16 rows with D % 8 == 0 (and C % 8 == 0): 16-byte vectors, the row's dy
// and y kept in registers between the reduction and the update.
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  const uint32_t* w = (const uint32_t*)&u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(w[e] << 16);
    f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ uint4 pack8f(const float* f) {
  uint4 u;
  u.x = pack2bf(f[0], f[1]);
  u.y = pack2bf(f[2], f[3]);
  u.z = pack2bf(f[4], f[5]);
  u.w = pack2bf(f[6], f[7]);
  return u;
}

template <int VPL>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_v(const bf16* dy, const bf16* y, const float* r,
                                                       const bf16* dres, bf16* dx, int64_t rows,
                                                       int D, const float* vez, const bf16* wg,
                                                       int Hkv, int C) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nv = D >> 3;
  const uint4* dyr = (const uint4*)(dy + row * D);
  const uint4* yr = (const uint4*)(y + row * D);
  const float* vz = vez ? vez + row * Hkv : nullptr;
  float g[VPL][8], yv[VPL][8];
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) {
      unpack8(dyr[v], g[k]);
      unpack8(yr[v], yv[k]);
      if (vz && 8 * v < C) {
        for (int kv = 0; kv < Hkv; ++kv) {
          float wgf[8];
          unpack8(*(const uint4*)(wg + (int64_t)kv * C + 8 * v), wgf);
#pragma unroll
          for (int e = 0; e < 8; ++e) g[k][e] += vz[kv] * wgf[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += g[k][e] * yv[k][e];
    }
  }
  const float m = wave_sum(acc) / (float)D;
  const float rr = r[row];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) {
      float o[8];
      if (dres) unpack8(((const uint4*)(dres + row * D))[v], o);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += rr * (g[k][e] - yv[k][e] * m);
      ((uint4*)(dx + row * D))[v] = pack8f(o);
    }
  }
}

hipError_t rmsnorm_bwd(const void* dy, const void* y, const float* r,
                       const void* dres, void* dx, int64_t rows, int D,
                       const float* vez, const void* wg, int Hkv, int C,
                       DType dt, hipStream_t s) {
  dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  // dy, y (and dres) in, dx out, r in
  const Work w(0.0, (double)rows * D * (dres ? 4 : 3) * (dt == BF16 ? 2 : 4) + rows * 4.0);
  const bool vec = dt == BF16 && D % 8 == 0 && D <= 64 * 8 * 4 && (!vez || C % 8 == 0);
  if (vec) {
    const int vpl = (int)cdiv(D / 8, 64);
#define RMSB(V)                                                                              \
  GK_LAUNCH(w, k_rmsnorm_bwd_v<V>, grid, block, 0, s, (const bf16*)dy, (const bf16*)y, r, \
                     (const bf16*)dres, (bf16*)dx, rows, D, vez, (const bf16*)wg, Hkv, C)
    if (vpl == 1) RMSB(1);
    else if (vpl == 2) RMSB(2);
    else if (vpl == 3) RMSB(3);
    else RMSB(4);
#undef RMSB
  } else if (dt == BF16)
    GK_LAUNCH(w, k_rmsnorm_bwd<bf16>, grid, block, 0, s, (const bf16*)dy, (const bf16*)y, r,
                       (const bf16*)dres, (bf16*)dx, rows, D, vez, (const bf16*)wg, Hkv, C);
  else
    GK_LAUNCH(w, k_rmsnorm_bwd<float>, grid, block, 0, s, (const float*)dy, (const float*)y, r,
                       (const float*)dres, (float*)dx, rows, D, vez, (const float*)wg, Hkv, C);
  return hipGetLastError();
}

// ------------------------------------------------------ rotary + QK-norm
// One thread per rotation pair (j, j + hd/2) of a q or k head; the hd/2
// threads of a head are an aligned lane segment, so the norm's sum is a
// segment shuffle.  Threads past the end still shuffle (whole segments are
// out of range together) but neither load nor store.
template <typename Tv>
__global__ __launch_bounds__(256) void k_rope_qknorm_fwd(Tv* qkv, float* rq, float* rk,
                                                         const float2* cs, int64_t N, int T,
                                                         int H, int Hkv, int hd, float eps) {
  int half = hd >> 1, heads = H + Hkv;
  int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  bool valid = idx < N * heads * half;
  int64_t id = valid ? idx : 0;
  int j = (int)(id % half);
  int64_t rest = id / half;
  int hh = (int)(rest % heads);
  int64_t n = rest / heads;
  int t = (int)(n % T);
  Tv* p = qkv + n * (int64_t)((H + 2 * Hkv) * hd) + (int64_t)hh * hd;
  float x1 = valid ? ld(p, j) : 0.f, x2 = valid ? ld(p, j + half) : 0.f;
  float2 c = cs[(int64_t)t * half + j];
  float y1 = x1 * c.x - x2 * c.y;
  float y2 = x1 * c.y + x2 * c.x;
  float ss = seg_sum(y1 * y1 + y2 * y2, half);
  float rr = 1.0f / sqrtf(ss / (float)hd + eps);
  if (valid) {
    st(p, j, y1 * rr);
    st(p, j + half, y2 * rr);
    if (j == 0) {
      if (hh < H) rq[n * H + hh] = rr;
      else rk[n * Hkv + (hh - H)] = rr;
    }
  }
}

template <typename Tv>
__global__ __launch_bounds__(256) void k_rope_qknorm_bwd(Tv* dqkv, const Tv* qkv, const float* rq,
                                                         const float* rk, const float2* cs,
                                                         int64_t N, int T, int H, int Hkv, int hd) {
  int half = hd >> 1, heads = H + Hkv;
  int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  bool valid = idx < N * heads * half;
  int64_t id = valid ? idx : 0;
  int j = (int)(id % half);
  int64_t rest = id / half;
  int hh = (int)(rest % heads);
  int64_t n = rest / heads;
  int t = (int)(n % T);
  int64_t off = n * (int64_t)((H + 2 * Hkv) * hd) + (int64_t)hh * hd;
  Tv* dp = dqkv + off;
  const Tv* yp = qkv + off;
  float g1 = valid ? ld(dp, j) : 0.f, g2 = valid ? ld(dp, j + half) : 0.f;
  float y1 = valid ? ld(yp, j) : 0.f, y2 = valid ? ld(yp, j + half) : 0.f;
  float m = seg_sum(g1 * y1 + g2 * y2, half) / (float)hd;
  float rr = valid ? (hh < H ? rq[n * H + hh] : rk[n * Hkv + (hh - H)]) : 0.f;
  float a1 = rr * (g1 - y1 * m), a2 = rr * (g2 - y2 * m);
  float2 c = cs[(int64_t)t * half + j];
  if (valid) {   // inverse rotation (angle -theta)
    st(dp, j, a1 * c.x + a2 * c.y);
    st(dp, j + half, -a1 * c.y + a2 * c.x);
  }
}

// bf16, hd % 8 == 0: each thread rotates 4 consecutive pairs (8-byte loads of
// x[4j..4j+3] and x[hd/2 + 4j..]); hd/8 threads per head form the segment.
__device__ __forceinline__ void unpack4(uint2 u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xFFFF0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ uint2 pack4f(const float* f) {
  uint2 u;
  u.x = pack2bf(f[0], f[1]);
  u.y = pack2bf(f[2], f[3]);
  return u;
}

__global__ __launch_bounds__(256) void k_rope_qknorm_fwd_v(bf16* qkv, float* rq, float* rk,
                                                           const float2* cs, int64_t N, int T,
                                                           int H, int Hkv, int hd, float eps) {
  const int half = hd >> 1, lph = hd >> 3, heads = H + Hkv;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const bool valid = idx < N * heads * lph;
  const int64_t id = valid ? idx : 0;
  const int j4 = (int)(id % lph);
  const int64_t rest = id / lph;
  const int hh = (int)(rest % heads);
  const int64_t n = rest / heads;
  const int t = (int)(n % T);
  bf16* p = qkv + n * (int64_t)((H + 2 * Hkv) * hd) + (int64_t)hh * hd;
  float x1[4], x2[4];
  unpack4(*(const uint2*)(p + 4 * j4), x1);
  unpack4(*(const uint2*)(p + half + 4 * j4), x2);
  const float4* c4 = (const float4*)(cs + (int64_t)t * half + 4 * j4);
  const float4 ca = c4[0], cb = c4[1];                // (cos, sin) x 4
  const float c[4] = {ca.x, ca.z, cb.x, cb.z}, sn[4] = {ca.y, ca.w, cb.y, cb.w};
  float y1[4], y2[4], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y1[e] = x1[e] * c[e] - x2[e] * sn[e];
    y2[e] = x1[e] * sn[e] + x2[e] * c[e];
    ss += y1[e] * y1[e] + y2[e] * y2[e];
  }
  ss = seg_sum(ss, lph);
  const float rr = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) { y1[e] *= rr; y2[e] *= rr; }
  if (valid) {
    *(uint2*)(p + 4 * j4) = pack4f(y1);
    *(uint2*)(p + half + 4 * j4) = pack4f(y2);
    if (j4 == 0) {
      if (hh < H) rq[n * H + hh] = rr;
      else rk[n * Hkv + (hh - H)] = rr;
    }
  }
}

__global__ __launch_bounds__(256) void k_rope_qknorm_bwd_v(bf16* dqkv, const bf16* qkv,
                                                           const float* rq, const float* rk,
                                                           const float2* cs, int64_t N, int T,
                                                           int H, int Hkv, int hd) {
  const int half = hd >> 1, lph = hd >> 3, heads = H + Hkv;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const bool valid = idx < N * heads * lph;
  const int64_t id = valid ? idx : 0;
  const int j4 = (int)(id % lph);
  const int64_t rest = id / lph;
  const int hh = (int)(rest % heads);
  const int64_t n = rest / heads;
  const int t = (int)(n % T);
  const int64_t off = n * (int64_t)((H + 2 * Hkv) * hd) + (int64_t)hh * hd;
  bf16* dp = dqkv + off;
  const bf16* yp = qkv + off;
  float g1[4], g2[4], y1[4], y2[4];
  unpack4(*(const uint2*)(dp + 4 * j4), g1);
  unpack4(*(const uint2*)(dp + half + 4 * j4), g2);
  unpack4(*(const uint2*)(yp + 4 * j4), y1);
  unpack4(*(const uint2*)(yp + half + 4 * j4), y2);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc += g1[e] * y1[e] + g2[e] * y2[e];
  const float m = seg_sum(acc, lph) / (float)hd;
  const float rr = hh < H ? rq[n * H + hh] : rk[n * Hkv + (hh - H)];
  const float4* c4 = (const float4*)(cs + (int64_t)t * half + 4 * j4);
  const float4 ca = c4[0], cb = c4[1];
  const float c[4] = {ca.x, ca.z, cb.x, cb.z}, sn[4] = {ca.y, ca.w, cb.y, cb.w};
  float o1[4], o2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {           // norm backward, then the inverse rotation
    const float a1 = rr * (g1[e] - y1[e] * m), a2 = rr * (g2[e] - y2[e] * m);
    o1[e] = a1 * c[e] + a2 * sn[e];
    o2[e] = -a1 * sn[e] + a2 * c[e];
  }
  if (valid) {
    *(uint2*)(dp + 4 * j4) = pack4f(o1);
    *(uint2*)(dp + half + 4 * j4) = pack4f(o2);
  }
}

hipError_t rope_qknorm_fwd(void* qkv, float* rq, float* rk, const float* cs, int B, int T,
                           int H, int Hkv, int hd, float eps, DType dt, hipStream_t s) {
  int64_t N = (int64_t)B * T;
  const Work w(0.0, (double)N * (H + Hkv) * (hd * 2.0 * (dt == BF16 ? 2 : 4) + 4));
  if (dt == BF16 && hd % 8 == 0) {
    const int64_t total = N * (H + Hkv) * (hd / 8);
    GK_LAUNCH(w, k_rope_qknorm_fwd_v, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                       (bf16*)qkv, rq, rk, (const float2*)cs, N, T, H, Hkv, hd, eps);
    return hipGetLastError();
  }
  int64_t total = N * (H + Hkv) * (hd / 2);
  dim3 grid((unsigned)cdiv(total, 256)), block(256);
  if (dt == BF16)
    GK_LAUNCH(w, k_rope_qknorm_fwd<bf16>, grid, block, 0, s, (bf16*)qkv, rq, rk,
                       (const float2*)cs, N, T, H, Hkv, hd, eps);
  else
    GK_LAUNCH(w, k_rope_qknorm_fwd<float>, grid, block, 0, s, (float*)qkv, rq, rk,
                       (const float2*)cs, N, T, H, Hkv, hd, eps);
  return hipGetLastError();
}

hipError_t rope_qknorm_bwd(void* dqkv, const void* qkv, const float* rq, const float* rk,
                           const float* cs, int B, int T, int H, int Hkv, int hd, DType dt,
                           hipStream_t s) {
  int64_t N = (int64_t)B * T;
  const Work w(0.0, (double)N * (H + Hkv) * (hd * 3.0 * (dt == BF16 ? 2 : 4) + 4));
  if (dt == BF16 && hd % 8 == 0) {
    const int64_t total = N * (H + Hkv) * (hd / 8);
    GK_LAUNCH(w, k_rope_qknorm_bwd_v, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                       (bf16*)dqkv, (const bf16*)qkv, rq, rk, (const float2*)cs, N, T, H, Hkv, hd);
    return hipGetLastError();
  }
  int64_t total = N * (H + Hkv) * (hd / 2);
  dim3 grid((unsigned)cdiv(total, 256)), block(256);
  if (dt == BF16)
    GK_LAUNCH(w, k_rope_qknorm_bwd<bf16>, grid, block, 0, s, (bf16*)dqkv, (const bf16*)qkv,
                       rq, rk, (const float2*)cs, N, T, H, Hkv, hd);
  else
    GK_LAUNCH(w, k_rope_qknorm_bwd<float>, grid, block, 0, s, (float*)dqkv, (const float*)qkv,
                       rq, rk, (const float2*)cs, N, T, H, Hkv, hd);
  return hipGetLastError();
}

// -------------------------------------------------------- value embedding
// One block per token.  Wave w computes the gates of KV heads w, w+4, ...
// One wavefront per token (4 per block): the Hkv gates (3 sigmoid of a C-long
// dot product, wave reductions), then v += g E[tok] over the Hkv hd values in
// passes of 256 (lane: 4 consecutive values of one head).
template <typename Tv>
__global__ __launch_bounds__(256) void k_ve_fwd(const int32_t* tok, int T, int64_t N, const Tv* h,
                                                int D, const Tv* wg, int C, const Tv* E, Tv* qkv,
                                                int ldqkv, int voff, float* g, int Hkv, int hd) {
  __shared__ float gs[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = blockIdx.x * 4 + w;
  if (n >= N) return;
  const int id = tok[(n / T) * (T + 1) + n % T];
  for (int kv = 0; kv < Hkv; ++kv) {
    float acc = 0.f;
    for (int c = lane; c < C; c += 64) acc = fmaf(ld(h, n * D + c), ld(wg, (int64_t)kv * C + c), acc);
    acc = wave_sum(acc);
    if (lane == 0) {
      const float gv = 3.0f / (1.0f + expf(-acc));
      gs[w][kv] = gv;
      g[n * Hkv + kv] = gv;
    }
  }
  // the gates written by lane 0 are read by the whole wave: LDS is coherent
  // within the wave once the writes are issued (s_waitcnt before the reads)
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int W = Hkv * hd;
  for (int c0 = 0; c0 < W; c0 += 256) {
    const int col = c0 + 4 * lane;
    if (col >= W) continue;
    const float gv = gs[w][col / hd];
    const int64_t vi = n * ldqkv + voff + col, ei = (int64_t)id * W + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) st(qkv, vi + e, fmaf(gv, ld(E, ei + e), ld(qkv, vi + e)));
  }
}

hipError_t ve_fwd(const int32_t* tok, int B, int T, const void* h, int D, const void* wg, int C,
                  const void* E, void* qkv, int ldqkv, int voff, float* g, int Hkv, int hd,
                  DType dt, hipStream_t s) {
  const int64_t N = (int64_t)B * T;
  if (Hkv > 64 || hd % 4) return hipErrorInvalidValue;
  if (dt == BF16)
    GK_LAUNCH(Work(), k_ve_fwd<bf16>, dim3((unsigned)cdiv(N, 4)), dim3(256), 0, s, tok, T, N,
              (const bf16*)h, D, (const bf16*)wg, C, (const bf16*)E, (bf16*)qkv, ldqkv, voff, g,
              Hkv, hd);
  else
    GK_LAUNCH(Work(), k_ve_fwd<float>, dim3((unsigned)cdiv(N, 4)), dim3(256), 0, s, tok, T, N,
              (const float*)h, D, (const float*)wg, C, (const float*)E, (float*)qkv, ldqkv, voff,
              g, Hkv, hd);
  return hipGetLastError();
}

template <typename Tv, bool SCATTER>
__global__ __launch_bounds__(256) void k_ve_bwd(const int32_t* tok, int T, const Tv* dqkv,
                                                int ldqkv, int voff, const Tv* E, const float* g,
                                                float* vez, float* dE, int Hkv, int hd) {
  int64_t n = blockIdx.x;
  int id = tok[(n / T) * (T + 1) + n % T];
  int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int tot = Hkv * hd;
  for (int kv = w; kv < Hkv; kv += 4) {
    float gv = g[n * Hkv + kv];
    float acc = 0.f;
    for (int d = lane; d < hd; d += 64) {
      float dv = ld(dqkv, n * ldqkv + voff + kv * hd + d);
      acc += dv * ld(E, (int64_t)id * tot + kv * hd + d);
      if constexpr (SCATTER) atomicAdd(dE + (int64_t)id * tot + kv * hd + d, gv * dv);
    }
    acc = wave_sum(acc);
    if (lane == 0) vez[n * Hkv + kv] = acc * gv * (1.0f - gv / 3.0f);
  }
}

// vez[n, kv] = (dv . E[tok[n]])_kv g (1 - g/3): one wavefront per token, the
// Hkv*hd values in passes of 256 (lane: 4 consecutive columns), each head's
// dot product a reduction over its hd/4 lanes.
template <typename Tv>
__global__ __launch_bounds__(256) void k_ve_vez(const int32_t* tok, int T, int64_t N,
                                                const Tv* dqkv, int ldqkv, int voff, const Tv* E,
                                                const float* g, float* vez, int Hkv, int hd) {
  const int64_t n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const int id = tok[(n / T) * (T + 1) + n % T];
  const int W = Hkv * hd, seg = hd / 4;
  for (int c0 = 0; c0 < W; c0 += 256) {
    const int col = c0 + 4 * lane;
    float acc = 0.f;
    if (col < W) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = fmaf(ld(dqkv, n * ldqkv + voff + col + e), ld(E, (int64_t)id * W + col + e), acc);
    }
    acc = seg_sum(acc, seg);
    if (col < W && (lane % seg) == 0) {
      const int kv = col / hd;
      const float gv = g[n * Hkv + kv];
      vez[n * Hkv + kv] = acc * gv * (1.0f - gv / 3.0f);
    }
  }
}

hipError_t ve_vez(const int32_t* tok, int B, int T, const void* dqkv, int ldqkv, int voff,
                  const void* E, const float* g, float* vez, int Hkv, int hd, DType dt,
                  hipStream_t s) {
  const int64_t N = (int64_t)B * T;
  if (hd % 4 || hd / 4 > 64) return hipErrorInvalidValue;
  if (dt == BF16)
    GK_LAUNCH(Work(), k_ve_vez<bf16>, dim3((unsigned)cdiv(N, 4)), dim3(256), 0, s, tok, T, N,
              (const bf16*)dqkv, ldqkv, voff, (const bf16*)E, g, vez, Hkv, hd);
  else
    GK_LAUNCH(Work(), k_ve_vez<float>, dim3((unsigned)cdiv(N, 4)), dim3(256), 0, s, tok, T, N,
              (const float*)dqkv, ldqkv, voff, (const float*)E, g, vez, Hkv, hd);
  return hipGetLastError();
}

hipError_t ve_bwd(const int32_t* tok, int B, int T, const void* dqkv, int ldqkv, int voff,
                  const void* E, const float* g, float* vez, float* dE, int Hkv, int hd,
                  DType dt, hipStream_t s) {
  int64_t N = (int64_t)B * T;
  if (dt == BF16)
    GK_LAUNCH(Work(), (k_ve_bwd<bf16, true>), dim3((unsigned)N), dim3(256), 0, s, tok, T, (const bf16*)dqkv,
                       ldqkv, voff, (const bf16*)E, g, vez, dE, Hkv, hd);
  else
    GK_LAUNCH(Work(), (k_ve_bwd<float, true>), dim3((unsigned)N), dim3(256), 0, s, tok, T, (const float*)dqkv,
                       ldqkv, voff, (const float*)E, g, vez, dE, Hkv, hd);
  return hipGetLastError();
}

// dWg[kv, c] = sum_n vez[n, kv] h[n, c], in two deterministic stages.  Stage
// one: each block takes a fixed run of rows; its 256 threads are 8 row
// groups x 32 channels (the channels of a row are one coalesced read) and
// keep all Hkv gate gradients of their channel; the 8 row groups are added in
// order through LDS.  Stage two: one wavefront per output adds the blocks'
// partials with a fixed lane assignment and butterfly.
constexpr int kVeMaxKv = 16, kVeMaxCb = 2;     // Hkv <= 16, C <= 64 in this path
template <typename Tv>
__global__ __launch_bounds__(256) void k_ve_wgrad_part(const float* vez, const Tv* h, int D,
                                                       int64_t N, int Hkv, int C, int64_t rows,
                                                       float* part) {
  __shared__ float red[8][kVeMaxKv * kVeMaxCb * 32];
  const int rg = threadIdx.x >> 5, cc = threadIdx.x & 31;
  const int64_t n0 = blockIdx.x * rows, n1 = min(N, n0 + rows);
  float acc[kVeMaxKv][kVeMaxCb];
#pragma unroll
  for (int kv = 0; kv < kVeMaxKv; ++kv)
#pragma unroll
    for (int cb = 0; cb < kVeMaxCb; ++cb) acc[kv][cb] = 0.f;
  for (int64_t n = n0 + rg; n < n1; n += 8) {
    float hv[kVeMaxCb];
#pragma unroll
    for (int cb = 0; cb < kVeMaxCb; ++cb) {
      const int c = cc + 32 * cb;
      hv[cb] = c < C ? ld(h, n * D + c) : 0.f;
    }
#pragma unroll
    for (int kv = 0; kv < kVeMaxKv; ++kv) {
      if (kv >= Hkv) break;
      const float z = vez[n * Hkv + kv];
#pragma unroll
      for (int cb = 0; cb < kVeMaxCb; ++cb) acc[kv][cb] = fmaf(z, hv[cb], acc[kv][cb]);
    }
  }
#pragma unroll
  for (int kv = 0; kv < kVeMaxKv; ++kv)
#pragma unroll
    for (int cb = 0; cb < kVeMaxCb; ++cb) red[rg][(kv * kVeMaxCb + cb) * 32 + cc] = acc[kv][cb];
  __syncthreads();
  const int HC = Hkv * C;
  for (int t = threadIdx.x; t < HC; t += blockDim.x) {
    const int kv = t / C, c = t % C;
    const int slot = (kv * kVeMaxCb + c / 32) * 32 + c % 32;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) v += red[r][slot];
    part[(int64_t)blockIdx.x * HC + t] = v;
  }
}

// any Hkv, C: one block per output, a fixed-order block reduction
template <typename Tv>
__global__ __launch_bounds__(256) void k_ve_wgrad_any(const float* vez, const Tv* h, int D,
                                                      int64_t N, int Hkv, int C, float* dWg,
                                                      int accumulate) {
  __shared__ float red[4];
  const int o = blockIdx.x, kv = o / C, c = o % C;
  float acc = 0.f;
  for (int64_t n = threadIdx.x; n < N; n += blockDim.x) acc += vez[n * Hkv + kv] * ld(h, n * D + c);
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float v = (red[0] + red[1]) + (red[2] + red[3]);
    dWg[o] = accumulate ? dWg[o] + v : v;
  }
}

__global__ __launch_bounds__(64) void k_ve_wgrad_sum(const float* part, int nb, int HC,
                                                     float* dWg, int accumulate) {
  const int t = blockIdx.x, lane = threadIdx.x;
  float v = 0.f;
  for (int b = lane; b < nb; b += 64) v += part[(int64_t)b * HC + t];
  v = wave_sum(v);
  if (lane == 0) dWg[t] = accumulate ? dWg[t] + v : v;
}

size_t ve_wgrad_scratch_bytes(int Hkv, int C) { return (size_t)kVeWgradBlocks * Hkv * C * 4; }

hipError_t ve_wgrad(const float* vez, const void* h, int D, int64_t N, int Hkv, int C, float* dWg,
                    int accumulate, float* part, DType dt, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (Hkv > kVeMaxKv || C > 32 * kVeMaxCb) {
    if (dt == BF16)
      GK_LAUNCH(Work(), k_ve_wgrad_any<bf16>, dim3(Hkv * C), dim3(256), 0, s, vez,
                (const bf16*)h, D, N, Hkv, C, dWg, accumulate);
    else
      GK_LAUNCH(Work(), k_ve_wgrad_any<float>, dim3(Hkv * C), dim3(256), 0, s, vez,
                (const float*)h, D, N, Hkv, C, dWg, accumulate);
    return hipGetLastError();
  }
  const int nb = (int)std::min<int64_t>(kVeWgradBlocks, cdiv(N, 8));
  const int64_t rows = cdiv(N, nb);
  const int HC = Hkv * C;
  const Work w(0.0, (double)N * (C * (dt == BF16 ? 2 : 4) + Hkv * 4));
  if (dt == BF16)
    GK_LAUNCH(w, k_ve_wgrad_part<bf16>, dim3((unsigned)nb), dim3(256), 0, s, vez, (const bf16*)h,
              D, N, Hkv, C, rows, part);
  else
    GK_LAUNCH(w, k_ve_wgrad_part<float>, dim3((unsigned)nb), dim3(256), 0, s, vez,
              (const float*)h, D, N, Hkv, C, rows, part);
  GK_LAUNCH(Work(), k_ve_wgrad_sum, dim3((unsigned)HC), dim3(64), 0, s, part, nb, HC, dWg,
            accumulate);
  return hipGetLastError();
}

// ---------------------------------------------------------- cross-entropy
// Combine two (max, sum-of-exp) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

// One block per row: fp32 log-sum-exp over V (online max), the row loss,
// and optionally the bf16/fp32 softmax gradient (softmax - onehot) * scale.
template <typename TD>
__global__ __launch_bounds__(256) void k_ce(const float* z, int64_t rows, int V,
                                            const int32_t* tok, int tgtT, int direct, float* ell,
                                            float* lse_out, TD* dz, float scale, int64_t row0) {
  __shared__ float sm[4], ssum[4];
  int64_t row = blockIdx.x;
  const float* zr = z + row * (int64_t)V;
  const int64_t n = row0 + row;
  int tgt = direct ? tok[n] : tok[(n / tgtT) * (tgtT + 1) + n % tgtT + 1];
  float m = -INFINITY, s = 0.f;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float x = zr[v];
    if (x > m) {
      s = s * expf(m - x) + 1.0f;
      m = x;
    } else {
      s += expf(x - m);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; ssum[w] = s; }
  __syncthreads();
  float M = sm[0], S = ssum[0];
  for (int k = 1; k < 4; ++k) lse_merge(M, S, sm[k], ssum[k]);
  float L = M + logf(S);
  if (threadIdx.x == 0) {
    ell[row] = L - zr[tgt];
    lse_out[row] = L;
  }
  if (dz) {
    TD* dr = dz + row * (int64_t)V;
    for (int v = threadIdx.x; v < V; v += blockDim.x) {
      float p = expf(zr[v] - L);
      if (v == tgt) p -= 1.0f;
      st(dr, v, p * scale);
    }
  }
}

// Single pass over a logit row: 512 threads hold the row in registers (NV4
// float4 each, V = 2048 NV4), so the logits are read from HBM once; max and
// sum are exact two-step block reductions.
template <int NV4>
__global__ __launch_bounds__(512) void k_ce_reg(const float* z, int V, const int32_t* tok,
                                                int tgtT, int direct, float* ell, float* lse_out,
                                                bf16* dz, float scale, int64_t row0) {
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const float4* zr = (const float4*)(z + row * (int64_t)V);
  const int64_t n = row0 + row;
  const int tgt = direct ? tok[n] : tok[(n / tgtT) * (tgtT + 1) + n % tgtT + 1];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float4 v[NV4];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    v[k] = zr[k * 512 + threadIdx.x];
    m = fmaxf(m, fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w)));
  }
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) M = fmaxf(M, red[k]);
  __syncthreads();
  float sacc = 0.f;
#pragma unroll
  for (int k = 0; k < NV4; ++k)
    sacc += (expf(v[k].x - M) + expf(v[k].y - M)) + (expf(v[k].z - M) + expf(v[k].w - M));
  sacc = wave_sum(sacc);
  if (lane == 0) red[w] = sacc;
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) S += red[k];
  const float L = M + logf(S);
  if (threadIdx.x == 0) {
    ell[row] = L - z[row * (int64_t)V + tgt];
    lse_out[row] = L;
  }
  if (dz) {
    uint2* dr = (uint2*)(dz + row * (int64_t)V);
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      const int c = k * 512 + threadIdx.x;
      float p[4] = {expf(v[k].x - L), expf(v[k].y - L), expf(v[k].z - L), expf(v[k].w - L)};
      if ((tgt >> 2) == c) p[tgt & 3] -= 1.0f;
      uint2 u;
      u.x = pack2bf(p[0] * scale, p[1] * scale);
      u.y = pack2bf(p[2] * scale, p[3] * scale);
      dr[c] = u;
    }
  }
}

hipError_t ce_rows(const float* z, int64_t rows, int V, const int32_t* tok, int tgt_T,
                   int tgt_direct, float* ell, float* lse, void* dz, float grad_scale,
                   DType dt, hipStream_t s, int64_t row0) {
  if (rows <= 0) return hipSuccess;
  // logits read once, the gradient written once, per-row results
  const Work w(0.0, (double)rows * V * (4.0 + (dz ? (dt == BF16 ? 2 : 4) : 0)) + rows * 12.0);
  if (dt == BF16 && V % 2048 == 0 && V <= 32768 && ((uintptr_t)z & 15) == 0) {
    const int nv4 = V / 2048;
#define CEREG(K)                                                                             \
  GK_LAUNCH(w, k_ce_reg<K>, dim3((unsigned)rows), dim3(512), 0, s, z, V, tok, tgt_T,      \
                     tgt_direct, ell, lse, (bf16*)dz, grad_scale, row0)
    switch (nv4) {
      case 1: CEREG(1); break;
      case 2: CEREG(2); break;
      case 4: CEREG(4); break;
      case 8: CEREG(8); break;
      case 16: CEREG(16); break;
      default: goto generic;
    }
#undef CEREG
    return hipGetLastError();
  }
generic:
  if (dt == BF16)
    GK_LAUNCH(w, k_ce<bf16>, dim3((unsigned)rows), dim3(256), 0, s, z, rows, V, tok, tgt_T,
                       tgt_direct, ell, lse, (bf16*)dz, grad_scale, row0);
  else
    GK_LAUNCH(w, k_ce<float>, dim3((unsigned)rows), dim3(256), 0, s, z, rows, V, tok, tgt_T,
                       tgt_direct, ell, lse, (float*)dz, grad_scale, row0);
  return hipGetLastError();
}

// Fused lm_head + cross-entropy, second half.  k_ce_stats: one wave per row,
// lse = M + log(sum_t s_t exp(m_t - M)) with M = max_t m_t over the row's
// per-tile (m_t, s_t), summed per lane then across the wave in a fixed
// order; ell = lse - the target's logit.
__global__ __launch_bounds__(256) void k_ce_stats(const float2* __restrict__ stats, int ntn,
                                                  const float* __restrict__ zt, int64_t rows,
                                                  float* __restrict__ ell,
                                                  float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float2* st = stats + row * ntn;
  float m = -INFINITY;
  for (int t = lane; t < ntn; t += 64) m = fmaxf(m, st[t].x);
  const float M = wave_max(m);
  float sacc = 0.f;
  for (int t = lane; t < ntn; t += 64) {
    const float2 v = st[t];
    sacc += v.y * expf(v.x - M);
  }
  const float L = M + logf(wave_sum(sacc));
  if (lane == 0) {
    ell[row] = L - zt[row];
    lse[row] = L;
  }
}

// k_ce_grad: one 512-thread block per row; the softmax gradient from the
// stored bf16 e = exp(logit - m_t) and the row's lse, rescaled per tile by
// exp(m_t - lse) grad_scale into dz (which may be e itself: every thread
// reads its runs before writing them), minus grad_scale at the target.
__global__ __launch_bounds__(512) void k_ce_grad(const float2* __restrict__ stats, int ntn,
                                                 const float* __restrict__ lse_in, int V,
                                                 const int32_t* __restrict__ tok, int T,
                                                 int direct, const uint16_t* e, uint16_t* dz,
                                                 float scale) {
  __shared__ float ct[1024];
  const int64_t row = blockIdx.x;
  const float2* st = stats + row * ntn;
  const float L = lse_in[row];
  for (int t = threadIdx.x; t < ntn; t += 512) ct[t] = expf(st[t].x - L) * scale;
  __syncthreads();
  const int tgt = direct ? tok[row] : tok[(row / T) * (T + 1) + row % T + 1];
  const uint4* pe = (const uint4*)(e + row * (int64_t)V);
  uint4* p = (uint4*)(dz + row * (int64_t)V);
  // eight 16-byte runs per thread in flight before the first store (the
  // stores would otherwise hold every next load behind them)
  constexpr int U = 8;
  const int n8 = V / 8;
  for (int k0 = threadIdx.x; k0 < n8; k0 += 512 * U) {
    uint4 u[U];
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (k0 + 512 * i < n8) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)(pe + k0 + 512 * i));
        u[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int k = k0 + 512 * i;
      if (k >= n8) break;
      const float c = ct[(8 * k) >> 8];
      const uint32_t* wu = (const uint32_t*)&u[i];
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(wu[q] << 16) * c;
        f[2 * q + 1] = __uint_as_float(wu[q] & 0xFFFF0000u) * c;
      }
      if ((tgt >> 3) == k) f[tgt & 7] -= scale;
      uint4 o;
      o.x = pack2bf(f[0], f[1]);
      o.y = pack2bf(f[2], f[3]);
      o.z = pack2bf(f[4], f[5]);
      o.w = pack2bf(f[6], f[7]);
      // streaming stores: the 2 bytes per logit leave for HBM at once (the
      // weight-gradient product that reads them runs later)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w}, (u32x4*)(p + k));
    }
  }
}

hipError_t ce_fix(const float* stats, const float* zt, int64_t rows, int V, const int32_t* tok,
                  int tgt_T, int tgt_direct, float* ell, float* lse, const void* e, void* dz,
                  float grad_scale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V % 256 || V / 256 > 1024) return hipErrorInvalidValue;
  if (dz && !e) return hipErrorInvalidValue;
  if (!lse || (ell && !zt)) return hipErrorInvalidValue;
  const int ntn = V / 256;
  if (ell) {
    // stats read once, ell and lse written
    const Work w(0.0, (double)rows * (8.0 * ntn + 12.0));
    GK_LAUNCH(w, k_ce_stats, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
              (const float2*)stats, ntn, zt, rows, ell, lse);
  }
  if (dz) {
    // e read and the gradient written once
    const Work w(0.0, (double)rows * (8.0 * ntn + 4.0) + 4.0 * (double)rows * V);
    GK_LAUNCH(w, k_ce_grad, dim3((unsigned)rows), dim3(512), 0, s, (const float2*)stats, ntn,
              lse, V, tok, tgt_T, tgt_direct, (const uint16_t*)e, (uint16_t*)dz, grad_scale);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- reductions
// loss = mean(ell): one 1024-thread block, 16-byte loads, fp64 sums in a
// fixed order (per thread, then per wave, then the 16 wave sums in order)
__global__ __launch_bounds__(1024) void k_loss_reduce(const float* ell, int64_t N, float* loss_ws,
                                                      float* loss_out, int* flag) {
  __shared__ double red[16];
  double acc = 0.0;
  if (((uintptr_t)ell & 15) == 0) {
    const int64_t n4 = N / 4;
    for (int64_t i = threadIdx.x; i < n4; i += blockDim.x) {
      const float4 v = ((const float4*)ell)[i];
      acc += ((double)v.x + (double)v.y) + ((double)v.z + (double)v.w);
    }
    for (int64_t i = 4 * n4 + threadIdx.x; i < N; i += blockDim.x) acc += (double)ell[i];
  } else {
    for (int64_t i = threadIdx.x; i < N; i += blockDim.x) acc += (double)ell[i];
  }
  acc = wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) tot += red[k];
    float loss = (float)(tot / (double)N);
    *loss_ws = loss;
    if (loss_out) *loss_out = loss;
    *flag = isfinite(loss) ? 0 : 1;
  }
}

hipError_t loss_reduce(const float* ell, int64_t N, float* loss_ws, float* loss_out, int* flag,
                       hipStream_t s) {
  GK_LAUNCH(Work(0.0, 4.0 * N), k_loss_reduce, dim3(1), dim3(1024), 0, s, ell, N, loss_ws,
            loss_out, flag);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_eval_accum(const float* ell, const int32_t* tok, int rows,
                                                    int T, const int32_t* tb, double* acc,
                                                    int first) {
  __shared__ double rn[4], rb[4];
  int64_t n_tok = (int64_t)rows * T;
  double a = 0.0, b = 0.0;
  for (int64_t i = threadIdx.x; i < n_tok; i += blockDim.x) {
    a += (double)ell[i];
    b += (double)tb[tok[(i / T) * (T + 1) + i % T + 1]];
  }
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  if ((threadIdx.x & 63) == 0) { rn[threadIdx.x >> 6] = a; rb[threadIdx.x >> 6] = b; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double A = (rn[0] + rn[1]) + (rn[2] + rn[3]);
    double Bb = (rb[0] + rb[1]) + (rb[2] + rb[3]);
    if (first) { acc[0] = A; acc[1] = Bb; }
    else { acc[0] += A; acc[1] += Bb; }
  }
}

hipError_t eval_accum(const float* ell, const int32_t* tok, int rows, int T,
                      const int32_t* token_bytes, double* acc, int first, hipStream_t s) {
  GK_LAUNCH(Work(), k_eval_accum, dim3(1), dim3(256), 0, s, ell, tok, rows, T, token_bytes, acc,
                     first);
  return hipGetLastError();
}

__global__ void k_eval_finish(const double* acc, double* out) {
  if (threadIdx.x == 0) {
    out[0] = acc[0];
    out[1] = acc[1];
    out[2] = acc[0] / (0.69314718055994530942 * acc[1]);
  }
}

hipError_t eval_finish(const double* acc, double* out, hipStream_t s) {
  GK_LAUNCH(Work(), k_eval_finish, dim3(1), dim3(64), 0, s, acc, out);
  return hipGetLastError();
}

}  // namespace gk
