// Flash attention for head_dim 128 on gfx950 MFMA (bf16 in, fp32 softmax).
//
// Causal, sliding window W (key j visible from query i iff 0 <= i - j <= W),
// grouped KV heads (query head h reads KV head h / (H / Hkv)), scale
// 1/sqrt(128).  Exact: an online softmax over 64-key tiles; tiles with no
// visible pair are never loaded, tiles with every pair visible skip the mask.
//
// Forward: one workgroup = 2 waves = 128 queries of one (row, head); each
// wave owns 64 queries and keeps them in registers.  Scores are formed
// transposed (keys x queries, X = K tile, Y = Q), so every lane owns one
// query of each 16-query block and its running max / sum are lane-local
// after a 4-lane reduction.  P goes from the score accumulators straight
// into the P.V MFMA (V staged transposed, see attn_tiles.h); the output
// accumulator is O^T (head-dim x queries), so each lane stores 4 adjacent
// head-dim values.
#include <math.h>

#include "attn_mfma.h"
#include "attn_tiles.h"
#include "common.h"

namespace gk {
using namespace attn;

static constexpr int FWD_BQ = 128;      // queries per workgroup (2 waves x 64)
static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

// Inclusive key range [lo, hi] seen by queries [q_lo, q_hi] under window W.
__device__ __forceinline__ void key_range(int q_lo, int q_hi, int W, int& lo, int& hi) {
  lo = q_lo - W > 0 ? q_lo - W : 0;
  hi = q_hi;
}

__global__ __launch_bounds__(128, 1) void k_attn_fwd_mfma(const bf16* __restrict__ qkv,
                                                          bf16* __restrict__ o,
                                                          float* __restrict__ lse, int T, int H,
                                                          int Hkv, int W) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[TR * LDR];
  __shared__ __attribute__((aligned(16))) bf16 Vt[HD * LDT];

  const int nqb = (T + FWD_BQ - 1) / FWD_BQ;
  const int qblk = nqb - 1 - (int)blockIdx.x;          // long rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (H / Hkv);
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * HD;
  const bf16* rowbase = qkv + (int64_t)b * T * ldq;
  const bf16* kbase = rowbase + (int64_t)(H + kvh) * HD;
  const bf16* vbase = rowbase + (int64_t)(H + Hkv + kvh) * HD;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int q0 = qblk * FWD_BQ;
  const int qw = q0 + wave * 64;                       // this wave's first query
  const float sl2 = kLog2e / sqrtf((float)HD);        // scores in log2 units

  // this wave's 64 queries, as MFMA Y operands: qf[qb][ks]
  bf16x8_t qf[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int qi = qw + 16 * qb + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = qi < T ? *(const uint4*)(rowbase + (int64_t)qi * ldq + (int64_t)h * HD + 32 * ks + 8 * g)
                       : make_uint4(0, 0, 0, 0);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  float m[4], l[4];
  f32x4_t oacc[8][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) oacc[hb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  int klo, khi;
  key_range(q0, min(q0 + FWD_BQ, T) - 1, W, klo, khi);
  const int kt0 = klo / TR, kt1 = khi / TR;

  TileRegs<128> kr, vr;
  kr.load_rows(kbase, ldq, kt0 * TR, T);
  vr.load_patches(vbase, ldq, kt0 * TR, T);

  for (int kt = kt0; kt <= kt1; ++kt) {
    const int k0 = kt * TR;
    kr.store_rows(Ks);
    vr.store_patches_T(Vt);
    __syncthreads();
    if (kt < kt1) {                                    // prefetch the next tile
      kr.load_rows(kbase, ldq, k0 + TR, T);
      vr.load_patches(vbase, ldq, k0 + TR, T);
    }
    // pairs of this wave: queries [qw, qw+63], keys [k0, k0+63]
    const bool any = (qw + 63 >= k0) && (qw - (k0 + 63) <= W) && qw < T;
    const bool full = (qw >= k0 + 63) && (qw + 63 - k0 <= W);
    if (any) {
      f32x4_t s[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) s[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8_t kf = rfrag(Ks, 16 * kb + lr, ks, g);
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) s[kb][qb] = mfma(kf, qf[qb][ks], s[kb][qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int qi = qw + 16 * qb + lr;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = s[kb][qb][r] * sl2;
            if (!full) {
              const int d = qi - (k0 + 16 * kb + 4 * g + r);
              if (d < 0 || d > W) v = -INFINITY;
            }
            s[kb][qb][r] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m[qb], mx);
        const float ms = mn == -INFINITY ? 0.f : mn;   // row with nothing visible yet
        const float alpha = exp2f(m[qb] - ms);
        m[qb] = mn;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = exp2f(s[kb][qb][r] - ms);
            s[kb][qb][r] = p;
            ls += p;
          }
        l[qb] = l[qb] * alpha + ls;
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) oacc[hb][qb] *= alpha;
      }
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        bf16x8_t pf[4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) pf[qb] = pack8(s[2 * ch][qb], s[2 * ch + 1][qb]);
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) {
          const bf16x8_t vf = tfrag(Vt, 16 * hb + lr, ch, g);
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) oacc[hb][qb] = mfma(vf, pf[qb], oacc[hb][qb]);
        }
      }
    }
    __syncthreads();
  }

  // normalise and store: lane holds O[query][16 hb + 4 g + r]
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float lt = l[qb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int qi = qw + 16 * qb + lr;
    if (qi >= T) continue;
    const float inv = 1.0f / lt;
    bf16* orow = o + ((int64_t)b * T + qi) * (int64_t)H * HD + (int64_t)h * HD;
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      uint2 u;
      u.x = pack2bf(oacc[hb][qb][0] * inv, oacc[hb][qb][1] * inv);
      u.y = pack2bf(oacc[hb][qb][2] * inv, oacc[hb][qb][3] * inv);
      *(uint2*)(orow + 16 * hb + 4 * g) = u;
    }
    if (g == 0) lse[((int64_t)b * H + h) * T + qi] = (m[qb] + log2f(lt)) * kLn2;
  }
}

bool attn_mfma_supported(int T, int H, int Hkv, int hd) {
  return hd == HD && T >= 1 && H % Hkv == 0;
}

hipError_t attn_mfma_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv,
                         int hd, int W, hipStream_t s) {
  (void)hd;
  dim3 grid((T + FWD_BQ - 1) / FWD_BQ, H, B);
  hipLaunchKernelGGL(k_attn_fwd_mfma, grid, dim3(128), 0, s, (const bf16*)qkv, (bf16*)o, lse, T,
                     H, Hkv, W);
  return hipGetLastError();
}

bool attn_mfma_bwd_supported(int, int, int, int) { return false; }

size_t attn_mfma_bwd_scratch_bytes(int, int, int, int) { return 0; }

// The backward still runs on the generic kernels (see k_attn.hip).
hipError_t attn_mfma_bwd(const void*, const void*, const float*, const void*, void*, float*,
                         void*, int, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gk
