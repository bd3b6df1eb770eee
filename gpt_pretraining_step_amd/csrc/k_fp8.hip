// Tensor-wise FP8 casts for FP8 linear layers (the nanochat walkthrough,
// "3. precision management": Float8Linear with tensor-wise scaling).
//
// x (bf16 or fp32, [rows, cols]) -> q = fp8(clamp(x * s, -fmax, fmax)), s =
// fmax / max(amax, 1e-12), amax = max |x| over the whole tensor; OCP e4m3
// (fmax 448) or e5m2 (fmax 57344), rounded to nearest even by the
// hardware's packed conversions.  Two launches: per-block maxima of |x|,
// then the cast, whose every block re-reduces those maxima (a few KB, fixed
// order) so no device-wide synchronisation is needed.  The cast writes q
// row-major, its transpose, or both (a 64 x 64 tile passes through LDS), and
// s and 1/s.  HBM-bound: x is read twice (amax, then cast), each output
// written once.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

constexpr int kTile = 64;
constexpr int kMaxParts = 1024;

template <int FMT>
__device__ __forceinline__ float fp8_max() {
  return FMT == 0 ? 448.f : 57344.f;
}

// max of magnitudes that keeps a NaN
__device__ __forceinline__ float absmax(float m, float v) {
  const float a = fabsf(v);
  return (a > m || a != a) ? a : m;
}

__device__ __forceinline__ float block_absmax(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = absmax(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = absmax(r, red[i]);
  return r;
}

// 8 values of x from element i (16-byte aligned run)
__device__ __forceinline__ void load8(const bf16* x, int64_t i, float* v) {
  const uint4 u = *(const uint4*)(x + i);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* x, int64_t i, float* v) {
  const float4 a = *(const float4*)(x + i), b = *(const float4*)(x + i + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// 4 fp32 (already scaled and clamped) -> 4 fp8 codes, nearest even
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

}  // namespace

// per-block max |x| over 8-element runs, grid-stride, four runs in flight
// per thread
template <typename T>
__global__ __launch_bounds__(256) void k_fp8_amax(const T* __restrict__ x, int64_t n8,
                                                  float* __restrict__ part) {
  __shared__ float red[4];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(x, 8 * (i + u * stride), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = absmax(m, v[u][e]);
  }
  for (; i < n8; i += stride) {
    float v[8];
    load8(x, 8 * i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = absmax(m, v[e]);
  }
  m = block_absmax(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// grid (cdiv(rows, 64), cdiv(cols, 64)), 256 threads: thread t converts 16
// values of row r0 + t / 4, columns c0 + 16 (t % 4) ..
template <typename T, int FMT>
__global__ __launch_bounds__(256) void k_fp8_cast(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                  const float* __restrict__ part, int nparts,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ qt,
                                                  float* __restrict__ scales) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile][kTile + 16];
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) m = absmax(m, part[i]);
  const float amax = block_absmax(m, red);
  const float fmax = fp8_max<FMT>();
  const float s = fmax / (amax != amax ? amax : fmaxf(amax, 1e-12f));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    scales[0] = s;
    scales[1] = 1.f / s;
  }
  const int64_t r0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
  const int tr = threadIdx.x >> 2, tc = 16 * (threadIdx.x & 3);
  const int64_t r = r0 + tr, c = c0 + tc;
  uint4 out = make_uint4(0, 0, 0, 0);
  if (r < rows && c < cols) {
    float v[16];
    load8(x, r * cols + c, v);
    load8(x, r * cols + c + 8, v + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float y = v[e] * s;
      v[e] = y != y ? y : fminf(fmaxf(y, -fmax), fmax);
    }
    out.x = pack4<FMT>(v[0], v[1], v[2], v[3]);
    out.y = pack4<FMT>(v[4], v[5], v[6], v[7]);
    out.z = pack4<FMT>(v[8], v[9], v[10], v[11]);
    out.w = pack4<FMT>(v[12], v[13], v[14], v[15]);
    if (q) *(uint4*)(q + r * cols + c) = out;
  }
  if (!qt) return;
  // transpose through LDS: byte (row tr, column tc + e) -> tile[tc + e][tr]
  const uint32_t w[4] = {out.x, out.y, out.z, out.w};
#pragma unroll
  for (int e = 0; e < 16; ++e) tile[tc + e][tr] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  __syncthreads();
  // thread t writes 16 bytes of qt row c0 + t / 4 (= a column of x), from
  // x rows r0 + 16 (t % 4) ..
  const int64_t oc = c0 + tr, orow = r0 + tc;
  if (oc < cols && orow < rows) *(uint4*)(qt + oc * rows + orow) = *(const uint4*)&tile[tr][tc];
}

size_t fp8_cast_scratch_bytes() { return kMaxParts * sizeof(float); }

hipError_t fp8_cast(const void* x, int64_t rows, int64_t cols, DType dt, int fmt, void* q,
                    void* qt, float* scales, void* scratch, hipStream_t s) {
  const int64_t n8 = rows * cols / 8;
  // about 8 runs of 8 per thread (two rounds of four loads in flight)
  const int parts = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxParts, cdiv(n8, 8 * 256)));
  float* part = (float*)scratch;
  const double in_bytes = (double)rows * cols * (dt == BF16 ? 2 : 4);
  if (dt == BF16)
    GK_LAUNCH(Work(0.0, in_bytes), k_fp8_amax<bf16>, dim3(parts), dim3(256), 0, s,
              (const bf16*)x, n8, part);
  else
    GK_LAUNCH(Work(0.0, in_bytes), k_fp8_amax<float>, dim3(parts), dim3(256), 0, s,
              (const float*)x, n8, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)cdiv(rows, kTile), (unsigned)cdiv(cols, kTile));
  const Work w(0.0, in_bytes + (double)rows * cols * ((q ? 1 : 0) + (qt ? 1 : 0)) + 8.0);
  uint8_t* qo = (uint8_t*)q;
  uint8_t* qto = (uint8_t*)qt;
  if (dt == BF16) {
    if (fmt == 0)
      GK_LAUNCH(w, (k_fp8_cast<bf16, 0>), grid, dim3(256), 0, s, (const bf16*)x, rows, cols, part,
                parts, qo, qto, scales);
    else
      GK_LAUNCH(w, (k_fp8_cast<bf16, 1>), grid, dim3(256), 0, s, (const bf16*)x, rows, cols, part,
                parts, qo, qto, scales);
  } else {
    if (fmt == 0)
      GK_LAUNCH(w, (k_fp8_cast<float, 0>), grid, dim3(256), 0, s, (const float*)x, rows, cols,
                part, parts, qo, qto, scales);
    else
      GK_LAUNCH(w, (k_fp8_cast<float, 1>), grid, dim3(256), 0, s, (const float*)x, rows, cols,
                part, parts, qo, qto, scales);
  }
  return hipGetLastError();
}

}  // namespace gk
