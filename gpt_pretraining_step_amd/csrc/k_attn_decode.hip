// KV-cache decode attention for head_dim 128 on gfx950 MFMA.
//
// The inference engine of [nanochat] "6. inference engine" attends from the
// newest tokens of each sequence to its cached keys and values
// (flash_attn_with_kvcache).  Here: sequence b holds L_b cached positions
// (the Tq new tokens included, at L_b - Tq .. L_b - 1); query head h reads KV
// head h / G; key j is visible from the query at position p iff
// 0 <= p - j <= W (the training kernels' causal-window rule); scale
// 1 / sqrt(128).
//
// Work split ("split-K" over the keys): one workgroup per (sequence, KV
// head, group of up to 16 query slots, chunk of 64-key tiles).  The G x Tq
// queries of a KV head form one 16-column MFMA operand, so every key tile is
// read from HBM once for all of them.  Each of the 4 waves owns a private
// LDS slot for one K and one V tile (buffer loads straight into LDS) and
// walks every 4th tile of the chunk with its own online softmax; the 4
// states are merged through LDS, and the chunks' partial (max, sum, O) by a
// second kernel in a fixed order.  HBM-bound: the roofline is the cache
// bytes read once.
#include <math.h>

#include "attn_tiles.h"
#include "common.h"
#include "kernels.h"

namespace gk {
using namespace attn;

namespace {

constexpr int DW = 4;                     // waves per workgroup
constexpr int QS = 16;                    // query slots per workgroup
constexpr int PSTRIDE = 2 + HD;           // partial record: m, l, O[128]
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;

// One wave fills a [64][128] tile (the attention tiles' swizzled layout)
// from rows [row0, row0 + 64) of a matrix with row stride ld elements;
// rows at or past `rows` read as zeros.  16 loads of 1 KB (4 rows each).
__device__ __forceinline__ void wave_tile_dma(const bf16* base, int64_t ld, int rows, int row0,
                                              bf16* tile, int lane) {
  const int64_t lim = rows > 0 ? ((int64_t)(rows - 1) * ld + HD) * 2 : 0;
  const i32x4_t rsrc = make_rsrc(base, lim);
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)tile);
  const uint32_t ldb = (uint32_t)(ld * 2);
  const int p = lane & 15;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * i + (lane >> 4);
    const uint32_t voff = (uint32_t)(row0 + r) * ldb + 16u * (uint32_t)(p ^ dsw(r));
    dma16(rsrc, lds + 1024u * i, voff);
  }
}

}  // namespace

// grid: (chunks, Hkv * qgroups, B); 256 threads
__global__ __launch_bounds__(256, 1) void k_attn_decode(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ lens, bf16* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part, int Tq, int Tmax, int H, int Hkv, int W, int nchunks,
    float off2) {
  __shared__ __attribute__((aligned(1024))) bf16 kvbuf[DW][2][TR * HD];   // 128 KB

  const int chunk = blockIdx.x;
  const int qgroups = (int)gridDim.y / Hkv;
  const int kvh = (int)blockIdx.y / qgroups, qgrp = (int)blockIdx.y % qgroups;
  const int b = blockIdx.z;
  const int G = H / Hkv;
  const int nq = G * Tq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int L = min(max(lens[b], 0), Tmax);
  const float sl2 = kLog2eD / sqrtf((float)HD);

  // this lane's query slot (MFMA column lr)
  const int slot = qgrp * QS + lr;
  const bool qvalid = slot < nq;
  const int hq = kvh * G + (qvalid ? slot / Tq : 0);
  const int tq = qvalid ? slot % Tq : 0;
  const int pos = L - Tq + tq;
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qvalid)
      u = *(const uint4*)(q + (((int64_t)b * Tq + tq) * H + hq) * HD + 32 * ks + 8 * g);
    qf[ks] = __builtin_bit_cast(bf16x8_t, u);
  }

  const int64_t ldkv = (int64_t)Hkv * HD;
  const bf16* kbase = kc + (int64_t)b * Tmax * ldkv + (int64_t)kvh * HD;
  const bf16* vbase = vc + (int64_t)b * Tmax * ldkv + (int64_t)kvh * HD;
  // tiles holding keys some query of the block can see (keys [max(0, L - Tq
  // - W), L)), split evenly over the chunks
  const int tlo = max(0, L - Tq - W) / TR, thi = (L + TR - 1) / TR;
  const int per = (thi - tlo + nchunks - 1) / nchunks;
  const int t_begin = tlo + chunk * per;
  const int t_end = min(thi, t_begin + per);

  float m = -INFINITY, l = 0.f;
  f32x4_t oacc[8];
#pragma unroll
  for (int hb = 0; hb < 8; ++hb) oacc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16* Ks = kvbuf[wave][0];
  bf16* Vs = kvbuf[wave][1];
  for (int t = t_begin + wave; t < t_end; t += DW) {
    const int k0 = t * TR;
    wave_tile_dma(kbase, ldkv, L, k0, Ks, lane);
    wave_tile_dma(vbase, ldkv, L, k0, Vs, lane);
    dma_wait();
    __builtin_amdgcn_wave_barrier();
    // S[key][query] = K Q^T; lane: keys 16 kb + 4 g + r, query lr
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = mfma(dfrag_row(Ks, 16 * kb + lr, 0, g), qf[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) s[kb] = mfma(dfrag_row(Ks, 16 * kb + lr, ks, g), qf[ks], s[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + 16 * kb + 4 * g + r;
        const int d = pos - j;
        const bool vis = qvalid && j < L && d >= 0 && d <= W;
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
    // online softmax in log2 units (a fixed offset when the scores are
    // bounded), lane-local after a 4-lane max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      mx = fmaxf(mx, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float mn, alpha;
    if (off2 > 0.f) {
      mn = off2 / sl2;                    // raw-score units
      alpha = 1.f;
    } else {
      mn = fmaxf(m, mx);
      alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mn) * sl2);
    }
    const float off = mn == -INFINITY ? 0.f : mn * sl2;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -off));
        s[kb][r] = p;
        ls += p;
      }
    l = fmaf(l, alpha, ls);
    m = mn;
    if (alpha != 1.f) {
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) oacc[hb] *= alpha;
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const bf16x8_t pf = pack8(s[2 * ch], s[2 * ch + 1]);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb)
        oacc[hb] = mfma(dfrag_col(Vs, 16 * hb, 32 * ch + 4 * g, 32 * ch + 16 + 4 * g, lr), pf,
                        oacc[hb]);
    }
    // every lane's tr reads of this slot are done before the next tile's
    // loads overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
  float lt = l;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);

  // merge the 4 waves (fixed order) through LDS: per wave 16 (m, l) pairs
  // and O^T [128][16]
  __syncthreads();
  float* red = (float*)&kvbuf[0][0][0];               // [DW][16][PSTRIDE]
  float* mine = red + wave * QS * PSTRIDE;
  if (g == 0) {
    mine[lr * PSTRIDE] = m;
    mine[lr * PSTRIDE + 1] = lt;
  }
#pragma unroll
  for (int hb = 0; hb < 8; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[lr * PSTRIDE + 2 + 16 * hb + 4 * g + r] = oacc[hb][r];
  __syncthreads();
  // thread (slot = tid / 16, part = tid % 16) finishes 8 head dims of a slot
  const int tslot = threadIdx.x >> 4, tpart = threadIdx.x & 15;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < DW; ++w) M = fmaxf(M, red[(w * QS + tslot) * PSTRIDE]);
  float Lsum = 0.f, acc8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
#pragma unroll
  for (int w = 0; w < DW; ++w) {
    const float* rec = red + (w * QS + tslot) * PSTRIDE;
    const float mw = rec[0];
    const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw - M) * sl2);
    Lsum = fmaf(rec[1], f, Lsum);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = fmaf(rec[2 + 8 * tpart + e], f, acc8[e]);
  }
  const int tsl = qgrp * QS + tslot;
  if (tsl >= nq) return;
  const int thq = kvh * G + tsl / Tq, ttq = tsl % Tq;
  if (nchunks == 1) {
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    bf16* orow = o + (((int64_t)b * Tq + ttq) * H + thq) * HD + 8 * tpart;
    uint4 u;
    u.x = pack2bf(acc8[0] * inv, acc8[1] * inv);
    u.y = pack2bf(acc8[2] * inv, acc8[3] * inv);
    u.z = pack2bf(acc8[4] * inv, acc8[5] * inv);
    u.w = pack2bf(acc8[6] * inv, acc8[7] * inv);
    *(uint4*)orow = u;
    if (tpart == 0) lse[((int64_t)b * H + thq) * Tq + ttq] = (M * sl2 + log2f(Lsum)) * kLn2D;
    return;
  }
  float* rec = part + ((((int64_t)b * Hkv + kvh) * qgroups + qgrp) * nchunks + chunk) * QS * PSTRIDE +
               tslot * PSTRIDE;
  if (tpart == 0) {
    rec[0] = M;
    rec[1] = Lsum;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) rec[2 + 8 * tpart + e] = acc8[e];
}

// merge the chunks' partials of one (sequence, KV head, query group): 16
// threads per query slot, chunks in order
__global__ __launch_bounds__(256) void k_attn_decode_merge(const float* __restrict__ part,
                                                           bf16* __restrict__ o,
                                                           float* __restrict__ lse, int Tq, int H,
                                                           int Hkv, int qgroups, int nchunks) {
  const int kvh = (int)blockIdx.y / qgroups, qgrp = (int)blockIdx.y % qgroups;
  const int b = blockIdx.z;
  const int G = H / Hkv, nq = G * Tq;
  const int tslot = threadIdx.x >> 4, tpart = threadIdx.x & 15;
  const int tsl = qgrp * QS + tslot;
  if (tsl >= nq) return;
  const float sl2 = kLog2eD / sqrtf((float)HD);
  const float* base = part + (((int64_t)b * Hkv + kvh) * qgroups + qgrp) * nchunks * QS * PSTRIDE +
                      tslot * PSTRIDE;
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, base[(int64_t)c * QS * PSTRIDE]);
  float Lsum = 0.f, acc8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float* rec = base + (int64_t)c * QS * PSTRIDE;
    const float f = rec[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((rec[0] - M) * sl2);
    Lsum = fmaf(rec[1], f, Lsum);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = fmaf(rec[2 + 8 * tpart + e], f, acc8[e]);
  }
  const int thq = kvh * G + tsl / Tq, ttq = tsl % Tq;
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  bf16* orow = o + (((int64_t)b * Tq + ttq) * H + thq) * HD + 8 * tpart;
  uint4 u;
  u.x = pack2bf(acc8[0] * inv, acc8[1] * inv);
  u.y = pack2bf(acc8[2] * inv, acc8[3] * inv);
  u.z = pack2bf(acc8[4] * inv, acc8[5] * inv);
  u.w = pack2bf(acc8[6] * inv, acc8[7] * inv);
  *(uint4*)orow = u;
  if (tpart == 0) lse[((int64_t)b * H + thq) * Tq + ttq] = (M * sl2 + log2f(Lsum)) * kLn2D;
}

namespace {
struct DecodePlan {
  int qgroups, nchunks;
  int64_t kvrows;     // cache rows one sequence can have visible, at most
};
DecodePlan decode_plan(int B, int Tq, int H, int Hkv, int Tmax, int W) {
  DecodePlan d;
  d.qgroups = (H / Hkv * Tq + QS - 1) / QS;
  d.kvrows = std::min<int64_t>(Tmax, (int64_t)W + Tq);
  // live tiles of a sequence, at most (the window's start need not be aligned)
  const int64_t tiles = std::min<int64_t>((Tmax + TR - 1) / TR, (d.kvrows + TR - 1) / TR + 1);
  // enough workgroups for two rounds over the CUs, each with at least 4 tiles
  const int64_t pairs = (int64_t)B * Hkv * d.qgroups;
  const int64_t nc = std::min<int64_t>((512 + pairs - 1) / pairs, (tiles + 3) / 4);
  d.nchunks = (int)std::max<int64_t>(1, nc);
  return d;
}
}  // namespace

size_t attn_decode_scratch_bytes(int B, int Tq, int H, int Hkv, int Tmax, int W) {
  const DecodePlan d = decode_plan(B, Tq, H, Hkv, Tmax, W);
  if (d.nchunks == 1) return 0;
  return (size_t)B * Hkv * d.qgroups * d.nchunks * QS * PSTRIDE * sizeof(float);
}

hipError_t attn_decode(const void* q, const void* kc, const void* vc, const int32_t* lens,
                       void* o, float* lse, int B, int Tq, int Tmax, int H, int Hkv, int W,
                       float score_bound, void* scratch, hipStream_t s) {
  const DecodePlan d = decode_plan(B, Tq, H, Hkv, Tmax, W);
  if (d.nchunks > 1 && !scratch) return hipErrorInvalidValue;
  dim3 grid(d.nchunks, Hkv * d.qgroups, B);
  // visible keys and values read once (an upper bound: min(Tmax, W + Tq)
  // rows per sequence, since the lengths live on the device), queries read
  // and outputs written once
  const double kvbytes = 2.0 * B * (double)d.kvrows * Hkv * HD * 2;
  const double qo = 2.0 * B * (double)Tq * H * HD * 2 + 4.0 * B * H * Tq;
  GK_LAUNCH(Work(0.0, kvbytes + qo), k_attn_decode, grid, dim3(DW * 64), 0, s, (const bf16*)q,
            (const bf16*)kc, (const bf16*)vc, lens, (bf16*)o, lse, (float*)scratch, Tq, Tmax, H,
            Hkv, W, d.nchunks, score_bound > 0.f ? score_bound * kLog2eD : 0.f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || d.nchunks == 1) return e;
  GK_LAUNCH(Work(0.0, (double)B * Hkv * d.qgroups * d.nchunks * QS * PSTRIDE * 4 + qo),
            k_attn_decode_merge, dim3(1, Hkv * d.qgroups, B), dim3(256), 0, s,
            (const float*)scratch, (bf16*)o, lse, Tq, H, Hkv, d.qgroups, d.nchunks);
  return hipGetLastError();
}

}  // namespace gk
