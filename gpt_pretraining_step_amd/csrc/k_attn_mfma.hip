// Flash attention for head_dim 128 on gfx950 MFMA (bf16 in, fp32 softmax).
//
// Causal, sliding window W (key j visible from query i iff 0 <= i - j <= W),
// grouped KV heads (query head h reads KV head h / (H / Hkv)), scale
// 1/sqrt(128).  Exact: an online softmax over 64-key tiles; tiles with no
// visible pair are never loaded, tiles with every pair visible skip the mask.
//
// Forward: one workgroup = 4 waves = 128 queries of one (row, head); each
// wave owns 32 queries and keeps them in registers (two waves per SIMD fit).  Scores are formed
// transposed (keys x queries, X = K tile, Y = Q), so every lane owns one
// query of each 16-query block and its running max / sum are lane-local
// after a 4-lane reduction.  P goes from the score accumulators straight
// into the P.V MFMA (V staged transposed, see attn_tiles.h); the output
// accumulator is O^T (head-dim x queries), so each lane stores 4 adjacent
// head-dim values.
#include <math.h>

#include <type_traits>

#include "attn_mfma.h"
#include "attn_tiles.h"
#include "common.h"

namespace gk {
using namespace attn;

static constexpr int NW = 4;                   // waves per workgroup
static constexpr int QW = 32;                  // queries per wave (2 blocks of 16)
// forward: 32 queries per wave at two waves per SIMD (48 or 64 queries at
// one wave per SIMD halve the LDS reads per product but measured 6-25%
// slower: the second wave hides the softmax and the tile waits)
static constexpr int FWD_QW = 32;              // forward: queries per wave
static constexpr int FQB = FWD_QW / 16;        // forward: 16-query blocks per wave
static constexpr int FWD_OCC = 2;              // forward: workgroups per CU (launch bound)
static constexpr int FWD_BQ = NW * FWD_QW;     // forward: queries per workgroup
static constexpr int DQ_BQ = NW * QW;          // backward dQ: queries per workgroup
static constexpr bool kJointDKV = true;        // dK and dV in one pass (16 keys a wave)
static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;
static constexpr float kLazy = 8.0f;           // forward: offset lag allowed (log2 units)

// Inclusive key range [lo, hi] seen by queries [q_lo, q_hi] under window W.
__device__ __forceinline__ void key_range(int q_lo, int q_hi, int W, int& lo, int& hi) {
  lo = q_lo - W > 0 ? q_lo - W : 0;
  hi = q_hi;
}

// Block numbering of the attention grids: the dispatcher deals workgroups
// round-robin over the 8 XCDs (each with its own L2), so a 1-D grid of
// 8 ceil(nblk npair / 8) ids is renumbered to give each XCD a contiguous
// run of whole (row, head) pairs, each pair's nblk blocks in the order
// blk = nblk - 1, ..., 0.  The blocks of one pair then stream the same
// tiles through one L2 at about the same time.  False for padding ids.
__device__ __forceinline__ bool xcd_block(int nblk, int npair, int& pair, int& blk) {
  const int nb = nblk * npair;
  const int per_xcd = (nb + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= nb) return false;
  pair = logical / nblk;
  blk = nblk - 1 - logical % nblk;
  return true;
}

__host__ inline dim3 xcd_grid(int nblk, int npair) {
  const int64_t nb = (int64_t)nblk * npair;
  return dim3((unsigned)(8 * ((nb + 7) / 8)));
}

// BOUNDED: the caller guarantees |q . k| / sqrt(hd) <= bound for every pair
// (true after QK-norm: RMS-normalised rows have norm <= sqrt(hd)), passed as
// off2 = bound * log2(e).  Then p = 2^(s log2(e) / sqrt(hd) - off2) <= 1 for
// every score with one fixed offset, so the online max, the rescaling of the
// output and the lazy-offset logic all drop out (the row sums stay fp32 sums
// of the unrounded P).  Without a bound the offset follows the running
// maximum.
template <bool BOUNDED>
__global__ __launch_bounds__(256, FWD_OCC) void k_attn_fwd_mfma(const bf16* __restrict__ qkv,
                                                          bf16* __restrict__ o,
                                                          float* __restrict__ lse, int B, int T,
                                                          int H, int Hkv, int W, float off2) {
  // two stages of (K tile, V tile), filled by buffer loads straight into LDS
  __shared__ __attribute__((aligned(16))) bf16 kv[2][2][TR * HD];

  // which (row, head) and query block, longest first, XCD-contiguous
  const int nqb = (T + FWD_BQ - 1) / FWD_BQ;
  int pair, qblk;
  if (!xcd_block(nqb, H * B, pair, qblk)) return;
  const int h = pair % H, b = pair / H;
  const int kvh = h / (H / Hkv);
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * HD;
  const bf16* rowbase = qkv + (int64_t)b * T * ldq;

  // the wave index is uniform: said so, the per-wave tile tests below are
  // scalar branches rather than per-lane selects
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int q0 = qblk * FWD_BQ;
  const int qw = q0 + wave * FWD_QW;                       // this wave's first query
  const float sl2 = kLog2e / sqrtf((float)HD);        // scores in log2 units

  const bf16* kbase = rowbase + (int64_t)(H + kvh) * HD;
  const bf16* vbase = rowbase + (int64_t)(H + Hkv + kvh) * HD;
  TileDma td;
  td.init(ldq, wave, lane);

  int klo, khi;
  key_range(q0, min(q0 + FWD_BQ, T) - 1, W, klo, khi);
  const int kt0 = klo / TR, kt1 = khi / TR;
  td.issue(kbase, T, kt0 * TR, kv[0][0], wave);
  td.issue(vbase, T, kt0 * TR, kv[0][1], wave);

  // this wave's queries as MFMA Y operands: qf[qb][ks]
  bf16x8_t qf[FQB][4];
#pragma unroll
  for (int qb = 0; qb < FQB; ++qb) {
    const int qi = qw + 16 * qb + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = qi < T ? *(const uint4*)(rowbase + (int64_t)qi * ldq + (int64_t)h * HD + 32 * ks + 8 * g)
                       : make_uint4(0, 0, 0, 0);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  // running max (raw score units) and sum per query
  float m[FQB], l[FQB];
  f32x4_t oacc[8][FQB];
#pragma unroll
  for (int qb = 0; qb < FQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) oacc[hb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // S = K Q^T for one stage, softmax, O += V^T P; the causal / window mask
  // unless every pair of the wave's tile is visible
  auto tile_body = [&](int k0, auto stc, bool full) {
    constexpr int st = decltype(stc)::value;
    const bf16* Ks = kv[st][0];
    const bf16* Vs = kv[st][1];
    f32x4_t s[4][FQB];
    // contraction step outermost: 4 FQB independent accumulators per step
    // keep the matrix pipeline busy between dependent products
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t kf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[kb] = dfrag_row(Ks, 16 * kb + lr, ks, g);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < FQB; ++qb)
          s[kb][qb] = mfma(kf[kb], qf[qb][ks],
                           ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : s[kb][qb]);
    }
    // mask (tiles on the diagonal or the window edge only: a wave-uniform
    // branch between two copies of the loop)
    if (!full) {
      // d = query - key from one per-tile base
      const int base = qw + lr - 4 * g - k0;
#pragma unroll
      for (int qb = 0; qb < FQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = base + (16 * qb - 16 * kb - r);
            s[kb][qb][r] = (unsigned)d > (unsigned)W ? -INFINITY : s[kb][qb][r];
          }
    }
    if constexpr (BOUNDED) {
#pragma unroll
      for (int qb = 0; qb < FQB; ++qb) {
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], sl2, -off2));
            s[kb][qb][r] = p;
            ls += p;
          }
        l[qb] += ls;
      }
    } else {
    bool grew = false;
    float alpha[FQB];
#pragma unroll
    for (int qb = 0; qb < FQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(s[kb][qb][0], s[kb][qb][1]), fmaxf(s[kb][qb][2], s[kb][qb][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // The exponent offset m moves only when the tile's maximum exceeds it
      // by more than kLazy (log2 units), or on the first visible tile: the
      // probabilities then stay below 2^kLazy, exact in fp32 and in bf16's
      // relative precision, and the output is rescaled rarely.
      const bool up = m[qb] == -INFINITY ? mx > -INFINITY : (mx - m[qb]) * sl2 > kLazy;
      const float mn = up ? mx : m[qb];
      grew |= up;
      const float off = mn == -INFINITY ? 0.f : mn * sl2;   // nothing visible yet: 0
      alpha[qb] = up ? __builtin_amdgcn_exp2f(fmaf(m[qb], sl2, -off)) : 1.f;
      m[qb] = mn;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], sl2, -off));
          s[kb][qb][r] = p;
          ls += p;
        }
      l[qb] = fmaf(l[qb], alpha[qb], ls);
    }
    // rescale the output only when some running max of the wave moved
    if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
      for (int qb = 0; qb < FQB; ++qb)
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) oacc[hb][qb] *= alpha[qb];
    }
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      bf16x8_t pf[FQB];
#pragma unroll
      for (int qb = 0; qb < FQB; ++qb) pf[qb] = pack8(s[2 * ch][qb], s[2 * ch + 1][qb]);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) {
        const bf16x8_t vf = dfrag_col(Vs, 16 * hb, 32 * ch + 4 * g, 32 * ch + 16 + 4 * g, lr);
#pragma unroll
        for (int qb = 0; qb < FQB; ++qb) oacc[hb][qb] = mfma(vf, pf[qb], oacc[hb][qb]);
      }
    }
  };

  // one key tile; the loop below is unrolled by two so every LDS address
  // names its stage statically (fragment addresses become per-lane bases
  // plus immediate offsets, no per-tile address arithmetic)
  auto tile = [&](int kt, auto stc) {
    const int k0 = kt * TR;
    constexpr int st = decltype(stc)::value;
    dma_wait();
    __syncthreads();                                   // stage st filled, stage st^1 free
    if (kt < kt1) {
      td.issue(kbase, T, k0 + TR, kv[st ^ 1][0], wave);
      td.issue(vbase, T, k0 + TR, kv[st ^ 1][1], wave);
    }
    // pairs of this wave: queries [qw, qw+31], keys [k0, k0+63]
    const bool any = (qw + FWD_QW - 1 >= k0) && (qw - (k0 + TR - 1) <= W) && qw < T;
    const bool full = (qw >= k0 + TR - 1) && (qw + FWD_QW - 1 - k0 <= W);
    if (!any) return;
    tile_body(k0, stc, full);
  };
  int kt = kt0;
  for (; kt + 1 <= kt1; kt += 2) {
    tile(kt, std::integral_constant<int, 0>());
    tile(kt + 1, std::integral_constant<int, 1>());
  }
  if (kt <= kt1) tile(kt, std::integral_constant<int, 0>());

  // normalise and store: lane holds O[query][16 hb + 4 g + r]
#pragma unroll
  for (int qb = 0; qb < FQB; ++qb) {
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
    const float off = BOUNDED ? off2 : m[qb] * sl2;
    if (g == 0) lse[((int64_t)b * H + h) * T + qi] = (off + log2f(lt)) * kLn2;
  }
}

bool attn_mfma_supported(int T, int H, int Hkv, int hd) {
  return hd == HD && T >= 1 && H % Hkv == 0;
}

hipError_t attn_mfma_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv,
                         int hd, int W, hipStream_t s, float score_bound) {
  (void)hd;
  const dim3 grid = xcd_grid((T + FWD_BQ - 1) / FWD_BQ, H * B);
  // 2 hd flops per visible pair for each of S = Q K^T and O = P V; q, k, v
  // read once, o and lse written once
  const double pairs = (double)B * H * visible_pairs(T, W), tok = (double)B * T;
  const Work w(4.0 * HD * pairs, tok * HD * 2 * (2.0 * H + 2 * Hkv) + tok * H * 4);
  if (score_bound > 0.f)
    GK_LAUNCH(w, k_attn_fwd_mfma<true>, grid, dim3(NW * 64), 0, s, (const bf16*)qkv, (bf16*)o,
              lse, B, T, H, Hkv, W, score_bound * kLog2e);
  else
    GK_LAUNCH(w, k_attn_fwd_mfma<false>, grid, dim3(NW * 64), 0, s, (const bf16*)qkv, (bf16*)o,
              lse, B, T, H, Hkv, W, 0.f);
  return hipGetLastError();
}

// ---------------------------------------------------------------- backward
//
// Delta_i = sum_d dO[i, d] O[i, d] per (row, head): 16 lanes per head row.
__global__ __launch_bounds__(256) void k_attn_delta(const bf16* __restrict__ o,
                                                    const bf16* __restrict__ dout,
                                                    float* __restrict__ delta, int T, int H,
                                                    int64_t rows) {
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t rh = gid >> 4;                        // (token, head) index
  const int part = gid & 15;
  const bool valid = rh < rows;
  const int64_t r = valid ? rh : 0;
  const uint4 a = *(const uint4*)(o + r * HD + part * 8);
  const uint4 d = *(const uint4*)(dout + r * HD + part * 8);
  const uint32_t* wa = (const uint32_t*)&a;
  const uint32_t* wd = (const uint32_t*)&d;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc += __uint_as_float(wa[e] << 16) * __uint_as_float(wd[e] << 16);
    acc += __uint_as_float(wa[e] & 0xFFFF0000u) * __uint_as_float(wd[e] & 0xFFFF0000u);
  }
  acc = seg_sum(acc, 16);
  if (valid && part == 0) {
    const int64_t n = r / H;                          // token = b*T + t
    const int hh = (int)(r % H);
    const int64_t b = n / T, t = n % T;
    delta[(b * H + hh) * T + t] = acc;
  }
}

// Backward of "RoPE then QK-norm" fused into the dQ / dK epilogues (used by
// the step; the kernel-level entry leaves it out).  One head row (hd = 128)
// sits in the MFMA output layout: lane (g, l16) holds x[16 hb + 4 g + r],
// hb < 8, r < 4 (the gradient w.r.t. the normalised q or k, already
// scaled).  It is rounded to bf16 as the unfused path stores it, then
// dx = rr (x - y mean(x y)) with y the saved normalised row and rr its
// 1/rms, then the rotation is undone: pairs (d, d + 64) are (hb, hb + 4) of
// the same lane.  The four lanes of a row (g = 0..3) finish the dot product
// with two shuffles.
struct NormBwdArgs {
  const float* rq;      // [B*T, H] 1/rms of the rotated q heads
  const float* rk;      // [B*T, Hkv]
  const float2* cs;     // [T, 64] (cos, sin)
};

__device__ __forceinline__ void norm_rope_bwd_row(float (&x)[8][4], const bf16* yrow, float rr,
                                                  const float2* csrow, int g, bool ok) {
  float y[8][4];
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < 8; ++hb) {
    const uint2 u = ok ? *(const uint2*)(yrow + 16 * hb + 4 * g) : make_uint2(0, 0);
    y[hb][0] = __uint_as_float(u.x << 16);
    y[hb][1] = __uint_as_float(u.x & 0xFFFF0000u);
    y[hb][2] = __uint_as_float(u.y << 16);
    y[hb][3] = __uint_as_float(u.y & 0xFFFF0000u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[hb][r] = bf2f(f2bf(x[hb][r]));
      acc = fmaf(x[hb][r], y[hb][r], acc);
    }
  }
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  const float m = acc / (float)HD;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float2 c = ok ? csrow[16 * hb + 4 * g + r] : make_float2(1.f, 0.f);
      const float a1 = rr * (x[hb][r] - y[hb][r] * m), a2 = rr * (x[hb + 4][r] - y[hb + 4][r] * m);
      x[hb][r] = a1 * c.x + a2 * c.y;
      x[hb + 4][r] = -a1 * c.y + a2 * c.x;
    }
  }
}

// dK, dV of 4 KPW keys of one KV head (4 waves x KPW keys), summed over the G
// query heads of the group and every 64-query tile that sees these keys.
// Scores are formed queries x keys (X = Q tile rows, Y = K in registers), so
// each lane owns one key; a 64-query tile is taken in halves of 16 NQB
// queries (NQB = 2 measured faster than whole tiles: fewer live scores),
// and P and dS of a half feed dV^T += dO^T P and dK^T += Q^T dS from
// registers, with the dO^T and Q^T fragments gathered by transposing LDS
// reads.
// MODE: 0 = dK and dV together, 1 = dK only, 2 = dV only (dV needs no dP,
// Delta or Q^T, dK no dO^T).  KPW: keys per wave, a multiple of 16.  At 32
// keys a wave the joint pass needs one wave per SIMD (both accumulators
// and the K and V fragments); at 16 it fits two, and S and P are formed
// once for both results.
template <int NQB, int MODE, bool FUSE, int KPW = 32>
__global__ __launch_bounds__(256, (MODE == 0 && KPW > 16) ? 1 : 2) void k_attn_bwd_dkv(const bf16* __restrict__ qkv,
                                                         const bf16* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ delta,
                                                         bf16* __restrict__ dqkv, int B, int T,
                                                         int H, int Hkv, int W, NormBwdArgs nb) {
  __shared__ __attribute__((aligned(16))) bf16 qd[2][2][TR * HD];   // stages of (Q, dO)
  __shared__ __attribute__((aligned(16))) float ldl[2][2][256];      // stages of (lse, delta)

  constexpr int KBN = KPW / 16, KV_BK = NW * KPW;   // key blocks per wave, keys per workgroup
  const int nkb = (T + KV_BK - 1) / KV_BK;
  int pair, kblk;
  if (!xcd_block(nkb, Hkv * B, pair, kblk)) return;
  // under the causal mask the first key blocks see the most queries: they
  // go first
  kblk = nkb - 1 - kblk;
  const int kvh = pair % Hkv, b = pair / Hkv;
  const int G = H / Hkv;
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const bf16* rowbase = qkv + (int64_t)b * T * ldq;
  const bf16* obase = dout + (int64_t)b * T * ldo;
  // the wave index is uniform: said so, the per-wave tile tests below are
  // scalar branches rather than per-lane selects
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int k0 = kblk * KV_BK;
  const int kw = k0 + KPW * wave;                     // this wave's first key
  const float sl2 = kLog2e / sqrtf((float)HD);
  constexpr bool DO_K = MODE != 2, DO_V = MODE != 1;

  // queries that see keys [k0, k0 + KV_BK - 1]: [k0, k0 + KV_BK - 1 + W]
  const int qhi = (int)min((int64_t)T - 1, (int64_t)k0 + KV_BK - 1 + W);
  const int qt0 = k0 / TR, nqt = qhi / TR - qt0 + 1;
  const int iters = G * nqt;

  TileDma tq, to;
  tq.init(ldq, wave, lane);
  to.init(ldo, wave, lane);
  auto issue = [&](int it, int st) {
    const int hh = kvh * G + it / nqt;
    const int qq = (qt0 + it % nqt) * TR;
    tq.issue(rowbase + (int64_t)hh * HD, T, qq, qd[st][0], wave);
    to.issue(obase + (int64_t)hh * HD, T, qq, qd[st][1], wave);
    if (wave == 0) {
      const int64_t li = ((int64_t)b * H + hh) * T;
      dma_vec64(lse + li, T, qq, ldl[st][0], lane);
      if constexpr (DO_K) dma_vec64(delta + li, T, qq, ldl[st][1], lane);
    }
  };
  issue(0, 0);

  bf16x8_t kf[KBN][4], vf[KBN][4];
#pragma unroll
  for (int kb = 0; kb < KBN; ++kb) {
    const int key = kw + 16 * kb + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int64_t off = (int64_t)key * ldq + 32 * ks + 8 * g;
      uint4 uk = key < T ? *(const uint4*)(rowbase + off + (int64_t)(H + kvh) * HD) : make_uint4(0, 0, 0, 0);
      kf[kb][ks] = __builtin_bit_cast(bf16x8_t, uk);
      if constexpr (DO_K) {
        uint4 uv = key < T ? *(const uint4*)(rowbase + off + (int64_t)(H + Hkv + kvh) * HD) : make_uint4(0, 0, 0, 0);
        vf[kb][ks] = __builtin_bit_cast(bf16x8_t, uv);
      }
    }
  }
  f32x4_t dk[8][KBN], dv[8][KBN];
#pragma unroll
  for (int hb = 0; hb < 8; ++hb)
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb) {
      dk[hb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dv[hb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // one query tile; unrolled by two below so LDS addresses name their stage
  // statically
  auto step = [&](int it, auto stc) {
    constexpr int st = decltype(stc)::value;
    const int q0 = (qt0 + it % nqt) * TR;
    dma_wait();
    __syncthreads();
    if (it + 1 < iters) issue(it + 1, st ^ 1);
    const bf16* Qs = qd[st][0];
    const bf16* Ds = qd[st][1];
    const float* Ls = ldl[st][0];
    const float* Dl = ldl[st][1];
#pragma unroll
    for (int hq = 0; hq < 4 / NQB; ++hq) {
      // pairs of this wave: queries [qa, qa + 16 NQB), keys [kw, kw + KPW)
      const int qa = q0 + 16 * NQB * hq;
      const bool any =
          (qa + 16 * NQB - 1 >= kw) && (qa - (kw + KPW - 1) <= W) && kw < T && qa < T;
      const bool full = (qa >= kw + KPW - 1) && (qa + 16 * NQB - 1 - kw <= W);
      if (!any) continue;
      f32x4_t s[NQB][KBN], dp[NQB][KBN];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int row = 16 * NQB * hq + 16 * qb + lr;
        const bf16x8_t qx0 = dfrag_row(Qs, row, 0, g);
        const bf16x8_t dx0 = DO_K ? dfrag_row(Ds, row, 0, g) : qx0;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          s[qb][kb] = mfma(qx0, kf[kb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
          if constexpr (DO_K) dp[qb][kb] = mfma(dx0, vf[kb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) {
          const bf16x8_t qx = dfrag_row(Qs, row, ks, g);
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb) s[qb][kb] = mfma(qx, kf[kb][ks], s[qb][kb]);
          if constexpr (DO_K) {
            const bf16x8_t dx = dfrag_row(Ds, row, ks, g);
#pragma unroll
            for (int kb = 0; kb < KBN; ++kb) dp[qb][kb] = mfma(dx, vf[kb][ks], dp[qb][kb]);
          }
        }
      }
      // P = exp(S - lse), dS = P (dP - Delta); lane: query qa+16qb+4g+r, key 16kb+lr
      if (!full) {                       // masked scores -> P = 0 (wave-uniform branch)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int d = qa + 16 * qb + 4 * g + r - (kw + 16 * kb + lr);
              s[qb][kb][r] = (unsigned)d > (unsigned)W ? -INFINITY : s[qb][kb][r];
            }
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qo = 16 * NQB * hq + 16 * qb + 4 * g;
        const f32x4_t L2 = *(const f32x4_t*)(Ls + qo) * kLog2e;
        const f32x4_t Dq = DO_K ? *(const f32x4_t*)(Dl + qo) : L2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int kb = 0; kb < KBN; ++kb) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], sl2, -L2[r]));
            s[qb][kb][r] = p;
            if constexpr (DO_K) dp[qb][kb][r] = p * (dp[qb][kb][r] - Dq[r]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < NQB / 2; ++c) {
        const int ch = (NQB / 2) * hq + c;                 // 32-query chunk of the tile
        const int ka = 32 * ch + 4 * g, kb2 = 32 * ch + 16 + 4 * g;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          if constexpr (DO_V) {
            const bf16x8_t pp = pack8(s[2 * c][kb], s[2 * c + 1][kb]);
#pragma unroll
            for (int hb = 0; hb < 8; ++hb)
              dv[hb][kb] = mfma(dfrag_col(Ds, 16 * hb, ka, kb2, lr), pp, dv[hb][kb]);
          }
          if constexpr (DO_K) {
            const bf16x8_t ps = pack8(dp[2 * c][kb], dp[2 * c + 1][kb]);
#pragma unroll
            for (int hb = 0; hb < 8; ++hb)
              dk[hb][kb] = mfma(dfrag_col(Qs, 16 * hb, ka, kb2, lr), ps, dk[hb][kb]);
          }
        }
      }
    }
    };
  int it = 0;
  for (; it + 2 <= iters; it += 2) {
    step(it, std::integral_constant<int, 0>());
    step(it + 1, std::integral_constant<int, 1>());
  }
  if (it < iters) step(it, std::integral_constant<int, 0>());
  // lane holds dK^T / dV^T [16hb + 4g + r][key 16kb + lr]
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int kb = 0; kb < KBN; ++kb) {
    const int key = kw + 16 * kb + lr;
    const bool ok = key < T;
    if constexpr (DO_K && FUSE) {          // every lane of the row takes part
      float x[8][4];
#pragma unroll
      for (int hb = 0; hb < 8; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[hb][r] = dk[hb][kb][r] * scale;
      const int64_t n = (int64_t)b * T + (ok ? key : 0);
      norm_rope_bwd_row(x, qkv + n * ldq + (int64_t)(H + kvh) * HD,
                        ok ? nb.rk[n * Hkv + kvh] : 0.f, nb.cs + (int64_t)(ok ? key : 0) * (HD / 2),
                        g, ok);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[hb][kb][r] = x[hb][r];
    }
    if (!ok) continue;
    bf16* krow = dqkv + ((int64_t)b * T + key) * ldq + (int64_t)(H + kvh) * HD;
    bf16* vrow = dqkv + ((int64_t)b * T + key) * ldq + (int64_t)(H + Hkv + kvh) * HD;
    const float ks = FUSE ? 1.f : scale;
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      if constexpr (DO_K) {
        uint2 uk;
        uk.x = pack2bf(dk[hb][kb][0] * ks, dk[hb][kb][1] * ks);
        uk.y = pack2bf(dk[hb][kb][2] * ks, dk[hb][kb][3] * ks);
        *(uint2*)(krow + 16 * hb + 4 * g) = uk;
      }
      if constexpr (DO_V) {
        uint2 uv;
        uv.x = pack2bf(dv[hb][kb][0], dv[hb][kb][1]);
        uv.y = pack2bf(dv[hb][kb][2], dv[hb][kb][3]);
        *(uint2*)(vrow + 16 * hb + 4 * g) = uv;
      }
    }
  }
}

// dQ of 128 queries of one head (4 waves x 32), over the key tiles they see.
// Scores keys x queries as in the forward; dS feeds dQ^T += K^T dS with the
// K^T fragments gathered from the K tile by transposing LDS reads.
template <bool FUSE>
__global__ __launch_bounds__(256, 2) void k_attn_bwd_dq(const bf16* __restrict__ qkv,
                                                        const bf16* __restrict__ dout,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ delta,
                                                        bf16* __restrict__ dqkv, int B, int T,
                                                        int H, int Hkv, int W, NormBwdArgs nb) {
  __shared__ __attribute__((aligned(16))) bf16 kv[2][2][TR * HD];   // stages of (K, V)

  const int nqb = (T + DQ_BQ - 1) / DQ_BQ;
  int pair, qblk;
  if (!xcd_block(nqb, H * B, pair, qblk)) return;
  const int h = pair % H, b = pair / H;
  const int kvh = h / (H / Hkv);
  const int64_t ldq = (int64_t)(H + 2 * Hkv) * HD, ldo = (int64_t)H * HD;
  const bf16* rowbase = qkv + (int64_t)b * T * ldq;
  const bf16* kbase = rowbase + (int64_t)(H + kvh) * HD;
  const bf16* vbase = rowbase + (int64_t)(H + Hkv + kvh) * HD;
  // the wave index is uniform: said so, the per-wave tile tests below are
  // scalar branches rather than per-lane selects
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int q0 = qblk * DQ_BQ;
  const int qw = q0 + wave * QW;
  const float sl2 = kLog2e / sqrtf((float)HD);

  TileDma td;
  td.init(ldq, wave, lane);
  int klo, khi;
  key_range(q0, min(q0 + DQ_BQ, T) - 1, W, klo, khi);
  const int kt0 = klo / TR, kt1 = khi / TR;
  td.issue(kbase, T, kt0 * TR, kv[0][0], wave);
  td.issue(vbase, T, kt0 * TR, kv[0][1], wave);

  bf16x8_t qf[2][4], df[2][4];
  float L2[2], Dq[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 16 * qb + lr;
    const bool ok = qi < T;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 uq = ok ? *(const uint4*)(rowbase + (int64_t)qi * ldq + (int64_t)h * HD + 32 * ks + 8 * g)
                    : make_uint4(0, 0, 0, 0);
      uint4 ud = ok ? *(const uint4*)(dout + ((int64_t)b * T + qi) * ldo + (int64_t)h * HD + 32 * ks + 8 * g)
                    : make_uint4(0, 0, 0, 0);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, uq);
      df[qb][ks] = __builtin_bit_cast(bf16x8_t, ud);
    }
    const int64_t li = ((int64_t)b * H + h) * T + qi;
    L2[qb] = ok ? lse[li] * kLog2e : INFINITY;
    Dq[qb] = ok ? delta[li] : 0.f;
  }
  f32x4_t dq[8][2];
#pragma unroll
  for (int hb = 0; hb < 8; ++hb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dq[hb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one key tile; unrolled by two below so LDS addresses name their stage
  // statically
  auto tile = [&](int kt, auto stc) {
    const int k0 = kt * TR;
    constexpr int st = decltype(stc)::value;
    dma_wait();
    __syncthreads();
    if (kt < kt1) {
      td.issue(kbase, T, k0 + TR, kv[st ^ 1][0], wave);
      td.issue(vbase, T, k0 + TR, kv[st ^ 1][1], wave);
    }
    const bf16* Ks = kv[st][0];
    const bf16* Vs = kv[st][1];
    const bool any = (qw + QW - 1 >= k0) && (qw - (k0 + TR - 1) <= W) && qw < T;
    const bool full = (qw >= k0 + TR - 1) && (qw + QW - 1 - k0 <= W);
    if (!any) return;
    f32x4_t s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8_t kx0 = dfrag_row(Ks, 16 * kb + lr, 0, g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma(kx0, qf[qb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
        const bf16x8_t kx = dfrag_row(Ks, 16 * kb + lr, ks, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma(kx, qf[qb][ks], s[kb][qb]);
      }
    }
    if (!full) {                         // masked scores -> P = 0 (wave-uniform branch)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = qw + 16 * qb + lr - (k0 + 16 * kb + 4 * g + r);
            s[kb][qb][r] = (unsigned)d > (unsigned)W ? -INFINITY : s[kb][qb][r];
          }
    }
    // lane: key 16kb + 4g + r, query 16qb + lr
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t dp[2];
      const bf16x8_t vx0 = dfrag_row(Vs, 16 * kb + lr, 0, g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) dp[qb] = mfma(vx0, df[qb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
        const bf16x8_t vx = dfrag_row(Vs, 16 * kb + lr, ks, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dp[qb] = mfma(vx, df[qb][ks], dp[qb]);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], sl2, -L2[qb]));
          s[kb][qb][r] = p * (dp[qb][r] - Dq[qb]);
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8_t ps[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) ps[qb] = pack8(s[2 * c][qb], s[2 * c + 1][qb]);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) {
        const bf16x8_t kt_ = dfrag_col(Ks, 16 * hb, 32 * c + 4 * g, 32 * c + 16 + 4 * g, lr);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dq[hb][qb] = mfma(kt_, ps[qb], dq[hb][qb]);
      }
    }
    };
  int kt = kt0;
  for (; kt + 1 <= kt1; kt += 2) {
    tile(kt, std::integral_constant<int, 0>());
    tile(kt + 1, std::integral_constant<int, 1>());
  }
  if (kt <= kt1) tile(kt, std::integral_constant<int, 0>());
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 16 * qb + lr;
    const bool ok = qi < T;
    float x[8][4];
#pragma unroll
    for (int hb = 0; hb < 8; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[hb][r] = dq[hb][qb][r] * scale;
    if constexpr (FUSE) {                  // every lane of the row takes part
      const int64_t n = (int64_t)b * T + (ok ? qi : 0);
      norm_rope_bwd_row(x, qkv + n * ldq + (int64_t)h * HD, ok ? nb.rq[n * H + h] : 0.f,
                        nb.cs + (int64_t)(ok ? qi : 0) * (HD / 2), g, ok);
    }
    if (!ok) continue;
    bf16* row = dqkv + ((int64_t)b * T + qi) * ldq + (int64_t)h * HD;
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      uint2 u;
      u.x = pack2bf(x[hb][0], x[hb][1]);
      u.y = pack2bf(x[hb][2], x[hb][3]);
      *(uint2*)(row + 16 * hb + 4 * g) = u;
    }
  }
}

bool attn_mfma_bwd_supported(int T, int H, int Hkv, int hd) {
  return attn_mfma_supported(T, H, Hkv, hd);
}

size_t attn_mfma_bwd_scratch_bytes(int, int, int, int) { return 0; }

hipError_t attn_mfma_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                         void* dqkv, float* delta, void*, int B, int T, int H, int Hkv, int hd,
                         int W, hipStream_t s, const float* nrq, const float* nrk,
                         const float* ncs, hipStream_t s2, hipEvent_t fork, hipEvent_t join,
                         hipStream_t s4, hipEvent_t join4) {
  (void)hd;
  const bool fuse = nrq && nrk && ncs;
  const NormBwdArgs nb{nrq, nrk, (const float2*)ncs};
  const int64_t rows = (int64_t)B * T * H;
  // Algorithmic work only: the backward's four products (dV = P^T dO,
  // dP = dO V^T, dK = dS^T Q, dQ = dS K) at 2 hd flops per visible pair
  // each, 8 hd in all, credited to the pass that produces each result (dK
  // pass: dP and dK; dV pass: dV; dQ pass: dQ).  The recomputed S (all
  // three passes) and the dQ pass's second dP are not counted.  Operands
  // read once, results written once.
  const double pairs = (double)B * H * visible_pairs(T, W), tok = (double)B * T;
  const double qkvo = tok * HD * 2 * (2.0 * H + 2 * Hkv), stats = (double)rows * 8;
  const Work wd(0.0, tok * H * HD * 2 * 2 + rows * 4.0);
  const Work wq(2.0 * HD * pairs, qkvo + stats + tok * H * HD * 2);
  GK_LAUNCH(wd, k_attn_delta, dim3((unsigned)cdiv(rows * 16, 256)), dim3(256), 0, s,
            (const bf16*)o, (const bf16*)dout, delta, T, H, rows);
  // the dQ and dV passes beside the dK pass: the three write disjoint parts
  // of dqkv and read only what Delta's pass and the forward left
  const bool two = s2 && fork && join;
  const hipStream_t sq = two ? s2 : s;
  const bool four = two && s4 && join4;
  const hipStream_t sv = four ? s4 : sq;
  if (two) {
    hipError_t e = hipEventRecord(fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s2, fork, 0);
    if (e == hipSuccess && four) e = hipStreamWaitEvent(s4, fork, 0);
    if (e != hipSuccess) return e;
  }
  // dK and dV in two passes (two waves per SIMD each; measured faster than
  // the one-wave-per-SIMD combined pass despite recomputing S)
  const dim3 gkv = xcd_grid((T + NW * 32 - 1) / (NW * 32), Hkv * B);       // 32 keys a wave
  const dim3 g16 = xcd_grid((T + NW * 16 - 1) / (NW * 16), Hkv * B);       // 16 keys a wave
  const Work wk(4.0 * HD * pairs, qkvo + stats + tok * Hkv * HD * 2);
  const Work wv(2.0 * HD * pairs, qkvo + stats / 2 + tok * Hkv * HD * 2);
  const dim3 gq = xcd_grid((T + DQ_BQ - 1) / DQ_BQ, H * B);
#define DKV_ARGS (const bf16*)qkv, (const bf16*)dout, lse, (const float*)delta, (bf16*)dqkv, B, T, H, Hkv, W, nb
  // dK (the longest pass) on the caller's stream, dQ and dV beside it on
  // streams of their own (or dV after dQ): 0.1 ms per d12 step each against
  // dV after dK on the caller's stream, and against dV after dQ
  const Work wkv(6.0 * HD * pairs, qkvo + stats + tok * Hkv * HD * 4);
  if (fuse && kJointDKV) {
    GK_LAUNCH(wq, k_attn_bwd_dq<true>, gq, dim3(NW * 64), 0, sq, DKV_ARGS);
    GK_LAUNCH(wkv, (k_attn_bwd_dkv<4, 0, true, 16>), g16, dim3(NW * 64), 0, s, DKV_ARGS);
  } else if (fuse) {
    GK_LAUNCH(wq, k_attn_bwd_dq<true>, gq, dim3(NW * 64), 0, sq, DKV_ARGS);
    GK_LAUNCH(wv, (k_attn_bwd_dkv<2, 2, false>), gkv, dim3(NW * 64), 0, sv, DKV_ARGS);
    GK_LAUNCH(wk, (k_attn_bwd_dkv<2, 1, true>), gkv, dim3(NW * 64), 0, s, DKV_ARGS);
  } else {
    GK_LAUNCH(wq, k_attn_bwd_dq<false>, gq, dim3(NW * 64), 0, sq, DKV_ARGS);
    GK_LAUNCH(wv, (k_attn_bwd_dkv<2, 2, false>), gkv, dim3(NW * 64), 0, sv, DKV_ARGS);
    GK_LAUNCH(wk, (k_attn_bwd_dkv<2, 1, false>), gkv, dim3(NW * 64), 0, s, DKV_ARGS);
  }
#undef DKV_ARGS
  if (two) {
    hipError_t e = hipEventRecord(join, s2);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, join, 0);
    if (e == hipSuccess && four) e = hipEventRecord(join4, s4);
    if (e == hipSuccess && four) e = hipStreamWaitEvent(s, join4, 0);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace gk
