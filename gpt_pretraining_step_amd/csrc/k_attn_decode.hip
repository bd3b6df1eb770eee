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
// read from HBM once for all of them.  Each of the 8 waves walks every 8th
// tile of the chunk with its own online softmax: the key rows go straight
// from memory into the registers that feed the score product, the value rows
// into the wave's LDS slot (buffer loads to LDS) for the transposing reads of
// the P V product.  The 8 states are merged through LDS; with several chunks
// each workgroup leaves its partial (max, sum, O) in scratch, and the last
// one to finish for a (sequence, KV head, query group) -- an arrival counter
// tells -- merges all of them in chunk order.  HBM-bound: the roofline is
// the cache bytes read once.
#include <math.h>

#include "attn_tiles.h"
#include "common.h"
#include "kernels.h"

namespace gk {
using namespace attn;

namespace {

constexpr int DW = 8;                     // waves per workgroup
constexpr int kTargetBlocks = 256;        // about one workgroup per CU
constexpr int QS = 16;                    // query slots per workgroup
constexpr int PSTRIDE = 2 + HD;           // partial record: m, l, O[128]
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;

// One wave fills a [64][128] tile (the attention tiles' swizzled layout)
// from rows [row0, row0 + 64) of a matrix with row stride ld elements;
// rows at or past `rows` read as zeros.  16 loads of 1 KB (4 rows each).
__device__ __forceinline__ void wave_tile_dma(const i32x4_t& rsrc, uint32_t ldb, int row0,
                                              bf16* tile, int lane) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)tile);
  const int p = lane & 15;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * i + (lane >> 4);
    const uint32_t voff = (uint32_t)(row0 + r) * ldb + 16u * (uint32_t)(p ^ dsw(r));
    dma16(rsrc, lds + 1024u * i, voff);
  }
}

// Merge `n` (m, l, O) records of one query slot (fixed order; this thread's
// 8 head dims at 8 * part): returns M, L and the 8 unnormalised sums.
struct Merged {
  float M, L, acc[8];
};
// Two floats of a record written by another workgroup of the running grid:
// an agent-scope atomic load (coherent across the chip's L2 caches).
__device__ __forceinline__ float2 coherent_load2(const float* p) {
  const uint64_t v = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(float2, v);
}
__device__ __forceinline__ void coherent_store2(float* p, float x, float y) {
  __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, make_float2(x, y)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool COHERENT>
__device__ __forceinline__ Merged merge_records(const float* rec0, int64_t step, int n, int part,
                                                float sl2) {
  Merged r;
  r.M = -INFINITY;
  for (int i = 0; i < n; ++i)
    r.M = fmaxf(r.M, COHERENT ? coherent_load2(rec0 + i * step).x : rec0[i * step]);
  r.L = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.acc[e] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float* rec = rec0 + i * step;
    float v[10];
    if constexpr (COHERENT) {
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const float2 w = coherent_load2(e == 0 ? rec : rec + 2 + 8 * part + 2 * (e - 1));
        v[2 * e] = w.x;
        v[2 * e + 1] = w.y;
      }
    } else {
      v[0] = rec[0];
      v[1] = rec[1];
      const float4 a = *(const float4*)(rec + 2 + 8 * part);
      const float4 b = *(const float4*)(rec + 6 + 8 * part);
      v[2] = a.x; v[3] = a.y; v[4] = a.z; v[5] = a.w;
      v[6] = b.x; v[7] = b.y; v[8] = b.z; v[9] = b.w;
    }
    const float f = v[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((v[0] - r.M) * sl2);
    r.L = fmaf(v[1], f, r.L);
#pragma unroll
    for (int e = 0; e < 8; ++e) r.acc[e] = fmaf(v[2 + e], f, r.acc[e]);
  }
  return r;
}

__device__ __forceinline__ void store_final(const Merged& r, bf16* orow, float* lse_at, int part,
                                            float sl2) {
  const float inv = r.L > 0.f ? 1.f / r.L : 0.f;
  uint4 u;
  u.x = pack2bf(r.acc[0] * inv, r.acc[1] * inv);
  u.y = pack2bf(r.acc[2] * inv, r.acc[3] * inv);
  u.z = pack2bf(r.acc[4] * inv, r.acc[5] * inv);
  u.w = pack2bf(r.acc[6] * inv, r.acc[7] * inv);
  *(uint4*)(orow + 8 * part) = u;
  if (part == 0) *lse_at = (r.M * sl2 + log2f(r.L)) * kLn2D;
}

}  // namespace

// grid: (chunks, Hkv * qgroups, B); 512 threads.  With more than one chunk:
// cnt, one arrival counter per (sequence, KV head, query group), zero on
// entry and left zero; part, per such triple and chunk 16 records.
__global__ __launch_bounds__(DW * 64, 1) void k_attn_decode(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ lens, bf16* __restrict__ o, float* __restrict__ lse,
    int* __restrict__ cnt, float* __restrict__ part, int Tq, int Tmax, int H, int Hkv, int W,
    int nchunks, float off2) {
  __shared__ __attribute__((aligned(1024))) bf16 vbuf[DW][TR * HD];   // 128 KB
  __shared__ int last_flag;

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
  const uint32_t ldb = (uint32_t)(ldkv * 2);
  const int64_t lim = L > 0 ? ((int64_t)(L - 1) * ldkv + HD) * 2 : 0;
  const bf16* kbase = kc + (int64_t)b * Tmax * ldkv + (int64_t)kvh * HD;
  const bf16* vbase = vc + (int64_t)b * Tmax * ldkv + (int64_t)kvh * HD;
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, (int)(uint32_t)lim, kRsrcWord3);
  const i32x4_t vrsrc = make_rsrc(vbase, lim);
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
  bf16* Vs = vbuf[wave];
  for (int t = t_begin + wave; t < t_end; t += DW) {
    const int k0 = t * TR;
    wave_tile_dma(vrsrc, ldb, k0, Vs, lane);
    // key fragments: row k0 + 16 kb + lr, head dims 32 ks + 8 g ..
    bf16x8_t kf[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[kb][ks] = __builtin_bit_cast(
            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                          krsrc, (int)((uint32_t)(k0 + 16 * kb + lr) * ldb + 64u * ks + 16u * g),
                          0, 0));
    // S[key][query] = K Q^T; lane: keys 16 kb + 4 g + r, query lr
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = mfma(kf[kb][0], qf[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) s[kb] = mfma(kf[kb][ks], qf[ks], s[kb]);
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
    dma_wait();
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const bf16x8_t pf = pack8(s[2 * ch], s[2 * ch + 1]);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb)
        oacc[hb] = mfma(dfrag_col(Vs, 16 * hb, 32 * ch + 4 * g, 32 * ch + 16 + 4 * g, lr), pf,
                        oacc[hb]);
    }
    // every lane's reads of the slot are done before the next tile's loads
    // overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
  float lt = l;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);

  // merge the 8 waves (fixed order) through LDS: per wave 16 (m, l) pairs
  // and O^T [128][16]
  __syncthreads();
  float* red = (float*)&vbuf[0][0];                   // [DW][16][PSTRIDE]
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
  // thread (slot = tid / 16, part = tid % 16) of the first 256 finishes 8
  // head dims of a slot
  const int tslot = (threadIdx.x >> 4) & (QS - 1), tpart = threadIdx.x & 15;
  const bool active = threadIdx.x < QS * 16 && qgrp * QS + tslot < nq;
  const int tsl = qgrp * QS + tslot;
  const int thq = kvh * G + tsl / Tq, ttq = tsl % Tq;
  bf16* orow = o + (((int64_t)b * Tq + ttq) * H + thq) * HD;
  float* lse_at = lse + ((int64_t)b * H + thq) * Tq + ttq;
  if (nchunks == 1) {
    if (active)
      store_final(merge_records<false>(red + tslot * PSTRIDE, QS * PSTRIDE, DW, tpart, sl2), orow,
                  lse_at, tpart, sl2);
    return;
  }
  const int64_t pair = ((int64_t)b * Hkv + kvh) * qgroups + qgrp;
  float* pbase = part + pair * nchunks * QS * PSTRIDE + tslot * PSTRIDE;
  // Publish this chunk's record with agent-scope stores, then count the
  // chunk with an acquire-release add at agent scope (one thread, after the
  // workgroup barrier that orders every wave's stores before it): the
  // release makes the record visible to whichever workgroup counts last,
  // and that workgroup's acquire orders its merge loads (agent-scope) after
  // every other chunk's release.  The last chunk to arrive merges all
  // records and sets the counter back to zero (the next launch sees it
  // through the kernel boundary).
  if (active) {
    const Merged r = merge_records<false>(red + tslot * PSTRIDE, QS * PSTRIDE, DW, tpart, sl2);
    float* rec = pbase + (int64_t)chunk * QS * PSTRIDE;
    if (tpart == 0) coherent_store2(rec, r.M, r.L);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      coherent_store2(rec + 2 + 8 * tpart + 2 * e, r.acc[2 * e], r.acc[2 * e + 1]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    last_flag = __hip_atomic_fetch_add(cnt + pair, 1, __ATOMIC_ACQ_REL,
                                       __HIP_MEMORY_SCOPE_AGENT) == nchunks - 1;
  __syncthreads();
  if (!last_flag) return;
  if (active)
    store_final(merge_records<true>(pbase, QS * PSTRIDE, nchunks, tpart, sl2), orow, lse_at,
                tpart, sl2);
  if (threadIdx.x == 0)
    __hip_atomic_store(cnt + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace {
struct DecodePlan {
  int qgroups, nchunks;
  int64_t kvrows;     // cache rows one sequence can have visible, at most
  int64_t pairs;      // (sequence, KV head, query group) triples
};
DecodePlan decode_plan(int B, int Tq, int H, int Hkv, int Tmax, int W) {
  DecodePlan d;
  d.qgroups = (H / Hkv * Tq + QS - 1) / QS;
  d.kvrows = std::min<int64_t>(Tmax, (int64_t)W + Tq);
  // live tiles of a sequence, at most (the window's start need not be aligned)
  const int64_t tiles = std::min<int64_t>((Tmax + TR - 1) / TR, (d.kvrows + TR - 1) / TR + 1);
  // about kTargetBlocks workgroups, each with at least 4 tiles
  d.pairs = (int64_t)B * Hkv * d.qgroups;
  const int64_t nc = std::min<int64_t>((kTargetBlocks + d.pairs - 1) / d.pairs, (tiles + 3) / 4);
  d.nchunks = (int)std::max<int64_t>(1, nc);
  return d;
}
}  // namespace

// with several chunks: arrival counters (one int per (sequence, KV head,
// query group), padded to 256 bytes), then the partial records
size_t counter_bytes(const DecodePlan& d) { return (d.pairs * 4 + 255) / 256 * 256; }

size_t attn_decode_counter_bytes(int B, int Tq, int H, int Hkv, int Tmax, int W) {
  const DecodePlan d = decode_plan(B, Tq, H, Hkv, Tmax, W);
  return d.nchunks == 1 ? 0 : counter_bytes(d);
}

size_t attn_decode_scratch_bytes(int B, int Tq, int H, int Hkv, int Tmax, int W) {
  const DecodePlan d = decode_plan(B, Tq, H, Hkv, Tmax, W);
  if (d.nchunks == 1) return 0;
  return counter_bytes(d) + (size_t)d.pairs * d.nchunks * QS * PSTRIDE * sizeof(float);
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
  int* cnt = (int*)scratch;
  float* part = d.nchunks > 1 ? (float*)((char*)scratch + counter_bytes(d)) : nullptr;
  GK_LAUNCH(Work(0.0, kvbytes + qo), k_attn_decode, grid, dim3(DW * 64), 0, s, (const bf16*)q,
            (const bf16*)kc, (const bf16*)vc, lens, (bf16*)o, lse, cnt, part, Tq, Tmax, H, Hkv,
            W, d.nchunks, score_bound > 0.f ? score_bound * kLog2eD : 0.f);
  return hipGetLastError();
}

}  // namespace gk
