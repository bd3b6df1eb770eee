// Causal sliding-window grouped-query attention of the GPT step on gfx950.
//
// Visible keys of query i: 0 <= i - j <= W.  Query head h reads KV head
// h / (H / Hkv).  Scale 1/sqrt(hd).  q, k, v are read from the fused qkv
// activation [B*T, (H + 2 Hkv) hd]; o is [B*T, H hd]; lse is [B, H, T].
//
// This file holds the generic wavefront-per-row kernels (any head_dim up to
// 128, fp32 or bf16).  The MFMA flash kernels for head_dim 128 live in
// k_attn_mfma.hip and are preferred when they apply.
#include <math.h>

#include "attn_mfma.h"
#include "common.h"
#include "kernels.h"

namespace gk {

// One wavefront per (b, h, i): lane d holds elements d and d + 64.
template <typename Tv>
__global__ __launch_bounds__(256) void k_attn_fwd_row(const Tv* qkv, Tv* o, float* lse, int B,
                                                      int T, int H, int Hkv, int hd, int W) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (row >= (int64_t)B * H * T) return;
  const int i = (int)(row % T);
  const int h = (int)((row / T) % H);
  const int64_t b = row / ((int64_t)T * H);
  const int kvh = h / (H / Hkv);
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * hd;
  const Tv* qr = qkv + (b * T + i) * ldq + (int64_t)h * hd;
  const bool e0 = lane < hd, e1 = lane + 64 < hd;
  const float scale = 1.0f / sqrtf((float)hd);
  const float q0 = e0 ? ld(qr, lane) : 0.f, q1 = e1 ? ld(qr, lane + 64) : 0.f;
  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
  const int jlo = i - W > 0 ? i - W : 0;
  for (int j = jlo; j <= i; ++j) {
    const Tv* kr = qkv + (b * T + j) * ldq + (int64_t)(H + kvh) * hd;
    const Tv* vr = kr + (int64_t)Hkv * hd;
    float s = q0 * (e0 ? ld(kr, lane) : 0.f) + q1 * (e1 ? ld(kr, lane + 64) : 0.f);
    s = wave_sum(s) * scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn);
    const float p = expf(s - mn);
    l = l * al + p;
    a0 = a0 * al + p * (e0 ? ld(vr, lane) : 0.f);
    a1 = a1 * al + p * (e1 ? ld(vr, lane + 64) : 0.f);
    m = mn;
  }
  Tv* orow = o + (b * T + i) * (int64_t)H * hd + (int64_t)h * hd;
  const float inv = 1.0f / l;
  if (e0) st(orow, lane, a0 * inv);
  if (e1) st(orow, lane + 64, a1 * inv);
  if (lane == 0) lse[(b * H + h) * T + i] = m + logf(l);
}

// dq (one wavefront per query row); also stores Delta_i = sum_d dO o.
template <typename Tv>
__global__ __launch_bounds__(256) void k_attn_bwd_dq_row(const Tv* qkv, const Tv* o,
                                                         const float* lse, const Tv* dout,
                                                         Tv* dqkv, float* delta, int B, int T,
                                                         int H, int Hkv, int hd, int W) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (row >= (int64_t)B * H * T) return;
  const int i = (int)(row % T);
  const int h = (int)((row / T) % H);
  const int64_t b = row / ((int64_t)T * H);
  const int kvh = h / (H / Hkv);
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * hd;
  const int64_t ldo = (int64_t)H * hd;
  const bool e0 = lane < hd, e1 = lane + 64 < hd;
  const float scale = 1.0f / sqrtf((float)hd);
  const Tv* qr = qkv + (b * T + i) * ldq + (int64_t)h * hd;
  const Tv* orow = o + (b * T + i) * ldo + (int64_t)h * hd;
  const Tv* dor = dout + (b * T + i) * ldo + (int64_t)h * hd;
  const float q0 = e0 ? ld(qr, lane) : 0.f, q1 = e1 ? ld(qr, lane + 64) : 0.f;
  const float d0 = e0 ? ld(dor, lane) : 0.f, d1 = e1 ? ld(dor, lane + 64) : 0.f;
  const float dl = wave_sum(d0 * (e0 ? ld(orow, lane) : 0.f) + d1 * (e1 ? ld(orow, lane + 64) : 0.f));
  const float L = lse[(b * H + h) * T + i];
  if (lane == 0) delta[(b * H + h) * T + i] = dl;
  float g0 = 0.f, g1 = 0.f;
  const int jlo = i - W > 0 ? i - W : 0;
  for (int j = jlo; j <= i; ++j) {
    const Tv* kr = qkv + (b * T + j) * ldq + (int64_t)(H + kvh) * hd;
    const Tv* vr = kr + (int64_t)Hkv * hd;
    const float k0 = e0 ? ld(kr, lane) : 0.f, k1 = e1 ? ld(kr, lane + 64) : 0.f;
    const float s = wave_sum(q0 * k0 + q1 * k1) * scale;
    const float p = expf(s - L);
    const float dp = wave_sum(d0 * (e0 ? ld(vr, lane) : 0.f) + d1 * (e1 ? ld(vr, lane + 64) : 0.f));
    const float ds = p * (dp - dl);
    g0 += ds * k0;
    g1 += ds * k1;
  }
  Tv* dq = dqkv + (b * T + i) * ldq + (int64_t)h * hd;
  if (e0) st(dq, lane, g0 * scale);
  if (e1) st(dq, lane + 64, g1 * scale);
}

// dk, dv (one wavefront per key row of a KV head), summed over the G query
// heads of its group and the queries i in [j, j + W].
template <typename Tv>
__global__ __launch_bounds__(256) void k_attn_bwd_dkv_row(const Tv* qkv, const float* lse,
                                                          const Tv* dout, const float* delta,
                                                          Tv* dqkv, int B, int T, int H, int Hkv,
                                                          int hd, int W) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (row >= (int64_t)B * Hkv * T) return;
  const int j = (int)(row % T);
  const int kvh = (int)((row / T) % Hkv);
  const int64_t b = row / ((int64_t)T * Hkv);
  const int G = H / Hkv;
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * hd;
  const int64_t ldo = (int64_t)H * hd;
  const bool e0 = lane < hd, e1 = lane + 64 < hd;
  const float scale = 1.0f / sqrtf((float)hd);
  const Tv* kr = qkv + (b * T + j) * ldq + (int64_t)(H + kvh) * hd;
  const Tv* vr = kr + (int64_t)Hkv * hd;
  const float k0 = e0 ? ld(kr, lane) : 0.f, k1 = e1 ? ld(kr, lane + 64) : 0.f;
  const float v0 = e0 ? ld(vr, lane) : 0.f, v1 = e1 ? ld(vr, lane + 64) : 0.f;
  float gk0 = 0.f, gk1 = 0.f, gv0 = 0.f, gv1 = 0.f;
  const int ihi = (int64_t)j + W < T - 1 ? j + W : T - 1;
  for (int hg = 0; hg < G; ++hg) {
    const int h = kvh * G + hg;
    for (int i = j; i <= ihi; ++i) {
      const Tv* qr = qkv + (b * T + i) * ldq + (int64_t)h * hd;
      const Tv* dor = dout + (b * T + i) * ldo + (int64_t)h * hd;
      const float q0 = e0 ? ld(qr, lane) : 0.f, q1 = e1 ? ld(qr, lane + 64) : 0.f;
      const float d0 = e0 ? ld(dor, lane) : 0.f, d1 = e1 ? ld(dor, lane + 64) : 0.f;
      const float s = wave_sum(q0 * k0 + q1 * k1) * scale;
      const float p = expf(s - lse[(b * H + h) * T + i]);
      const float dp = wave_sum(d0 * v0 + d1 * v1);
      const float ds = p * (dp - delta[(b * H + h) * T + i]);
      gv0 += p * d0;
      gv1 += p * d1;
      gk0 += ds * q0;
      gk1 += ds * q1;
    }
  }
  Tv* dk = dqkv + (b * T + j) * ldq + (int64_t)(H + kvh) * hd;
  Tv* dv = dk + (int64_t)Hkv * hd;
  if (e0) { st(dk, lane, gk0 * scale); st(dv, lane, gv0); }
  if (e1) { st(dk, lane + 64, gk1 * scale); st(dv, lane + 64, gv1); }
}

hipError_t attn_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd,
                    int W, DType dt, hipStream_t s, float score_bound) {
  if (dt == BF16 && attn_mfma_supported(T, H, Hkv, hd))
    return attn_mfma_fwd(qkv, o, lse, B, T, H, Hkv, hd, W, s, score_bound);
  const int64_t rows = (int64_t)B * H * T;
  dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  if (dt == BF16)
    GK_LAUNCH(Work(), k_attn_fwd_row<bf16>, grid, block, 0, s, (const bf16*)qkv, (bf16*)o, lse, B,
                       T, H, Hkv, hd, W);
  else
    GK_LAUNCH(Work(), k_attn_fwd_row<float>, grid, block, 0, s, (const float*)qkv, (float*)o, lse,
                       B, T, H, Hkv, hd, W);
  return hipGetLastError();
}

size_t attn_bwd_scratch_bytes(int B, int T, int H, int hd) {
  size_t delta = (size_t)B * H * T * sizeof(float);
  return ((delta + 255) / 256) * 256 + attn_mfma_bwd_scratch_bytes(B, T, H, hd);
}

bool attn_bwd_fuses_norm(int T, int H, int Hkv, int hd, DType dt) {
  return dt == BF16 && attn_mfma_bwd_supported(T, H, Hkv, hd);
}

hipError_t attn_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                    void* dqkv, void* scratch, int B, int T, int H, int Hkv, int hd, int W,
                    DType dt, hipStream_t s, const float* nrq, const float* nrk,
                    const float* ncs, const Beside& beside) {
  float* delta = (float*)scratch;
  if (dt == BF16 && attn_mfma_bwd_supported(T, H, Hkv, hd)) {
    size_t dbytes = (((size_t)B * H * T * sizeof(float) + 255) / 256) * 256;
    return attn_mfma_bwd(qkv, o, lse, dout, dqkv, delta, (char*)scratch + dbytes, B, T, H, Hkv,
                         hd, W, s, nrq, nrk, ncs, beside.s2, beside.fork, beside.join,
                         beside.s4, beside.join4);
  }
  const int64_t rows = (int64_t)B * H * T;
  const int64_t krows = (int64_t)B * Hkv * T;
  if (dt == BF16) {
    GK_LAUNCH(Work(), k_attn_bwd_dq_row<bf16>, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, s,
                       (const bf16*)qkv, (const bf16*)o, lse, (const bf16*)dout, (bf16*)dqkv, delta,
                       B, T, H, Hkv, hd, W);
    GK_LAUNCH(Work(), k_attn_bwd_dkv_row<bf16>, dim3((unsigned)cdiv(krows, 4)), dim3(256), 0, s,
                       (const bf16*)qkv, lse, (const bf16*)dout, delta, (bf16*)dqkv, B, T, H, Hkv,
                       hd, W);
  } else {
    GK_LAUNCH(Work(), k_attn_bwd_dq_row<float>, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, s,
                       (const float*)qkv, (const float*)o, lse, (const float*)dout, (float*)dqkv,
                       delta, B, T, H, Hkv, hd, W);
    GK_LAUNCH(Work(), k_attn_bwd_dkv_row<float>, dim3((unsigned)cdiv(krows, 4)), dim3(256), 0, s,
                       (const float*)qkv, lse, (const float*)dout, delta, (float*)dqkv, B, T, H,
                       Hkv, hd, W);
  }
  return hipGetLastError();
}

}  // namespace gk
