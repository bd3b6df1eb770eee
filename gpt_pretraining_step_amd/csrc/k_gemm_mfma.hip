// bf16 MFMA GEMM for gfx950 (CDNA4), fp32 accumulation.
//
// Block tile BM x BN x 64 with four wavefronts in a 2 x 2 grid; every wave
// owns a (BM/2) x (BN/2) sub-tile built from 16x16 v_mfma_f32_16x16x32_bf16
// blocks.  Operands are staged through LDS in a K-contiguous layout
// ([rows][64 + 8 pad]); the next K-slice is fetched into registers while the
// current one is consumed (register double buffering, one LDS stage), so two
// blocks fit per CU.
//
// Operands whose contraction index is the slow one in memory (A of TN, B of
// NN and TN) are transposed on the way in: each thread loads a KB x 8 patch
// (KB rows of 16 bytes), transposes it in registers with byte permutes and
// writes one K-contiguous run per column.  No separate transpose kernel and
// no extra HBM traffic.  The patch-to-lane assignment keeps those stores free
// of LDS bank conflicts.
//
// The MFMA is issued with B as the first source, so each lane ends up holding
// four consecutive columns of one output row: the epilogue writes 8-byte
// (bf16) or 16-byte (fp32) vectors.
//
// Blocks are numbered so that consecutive tiles land on the same XCD (the
// dispatcher deals workgroups round-robin over the 8 XCDs, each with its own
// L2), and tiles are visited in column-major groups of 8 tile rows.
//
// Weight-gradient products (TN) have few output tiles and a long reduction
// (the tokens), so they split K; partial tiles go to fp32 scratch and a
// second kernel adds them in a fixed order (deterministic).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "gemm_epi.h"
#include "gemm_mfma.h"

namespace gk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

static constexpr int BK = 64;
static constexpr int LDK = BK + 8;     // LDS row stride (elements), 144 bytes

// LDS element offset of (row, k).  With the 144-byte row stride, fragment
// reads (16 consecutive rows, one 16-byte chunk) hit 16 distinct bank groups,
// and the transposing stores below are arranged so that 16 lanes fill one
// 128-byte row segment; the address stays affine in the row, so fragment
// reads use one base register plus immediate offsets.
__device__ __forceinline__ int lds_off(int row, int k) { return row * LDK + k; }

// Layout used when both operands are transposed on the way in (TN): the
// column-fastest lane order there gives fully coalesced 256-byte global
// reads, and an XOR swizzle of the 16-byte chunks by (row / 16) % 8 keeps
// its stores (lanes 8 rows apart) free of bank conflicts.
template <bool XS>
__device__ __forceinline__ int lds_at(int row, int k) {
  if constexpr (XS) return row * LDK + ((((k >> 3) ^ (row >> 4)) & 7) << 3) + (k & 7);
  else return lds_off(row, k);
}

// low / high 16-bit halves of two words packed into one word
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// ---------------------------------------------------------------- staging
// K-contiguous operand: global [rows][ld], tile rows r0.., k0..k0+63.
template <int R, int NT = 256, bool XS = false>
struct KRowStage {
  static constexpr int CH = R * 8 / NT;     // 16-byte chunks per thread
  uint4 v[CH];
  __device__ __forceinline__ void load(const bf16* g, int64_t ld, int64_t r0, int64_t rows,
                                       int64_t k0, int64_t K) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c >> 3, kc = c & 7;
      const int64_t gr = r0 + r, gk = k0 + kc * 8;
      // clamped (always valid) address, then zero the lanes out of range:
      // no branch around the load
      const bool ok = gr < rows && gk < K;
      const uint4 x = *(const uint4*)(g + (ok ? gr : 0) * ld + (ok ? gk : 0));
      v[i] = ok ? x : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16* s) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c >> 3, kc = c & 7;
      *(uint4*)(s + lds_at<XS>(r, kc * 8)) = v[i];
    }
  }
};

// MN-contiguous operand: global [K][ld] (row index = k), tile columns r0..,
// k0..k0+63.  Each thread owns a KB x 8 patch.  Consecutive threads take
// consecutive k-blocks of the same 8 columns, so a load instruction reads
// 128-byte row segments and a store instruction fills 128-byte runs of one
// LDS row.
template <int R, int NT = 256, bool XS = false>
struct KColStage {
  static constexpr int NCB = R / 8;                 // 8-wide column blocks
  static constexpr int KB = 64 * NCB / NT;          // k rows per patch (8 or 4)
  static constexpr int NKB = 64 / KB;               // k-blocks per K-slice
  static_assert(KB == 8 || KB == 4, "tile width");
  uint4 v[KB];
  __device__ __forceinline__ void load(const bf16* g, int64_t ld, int64_t r0, int64_t rows,
                                       int64_t k0, int64_t K) {
    const int kb = XS ? threadIdx.x / NCB : threadIdx.x % NKB;
    const int cb = XS ? threadIdx.x % NCB : threadIdx.x / NKB;
    const int64_t col = r0 + cb * 8;
#pragma unroll
    for (int r = 0; r < KB; ++r) {
      const int64_t gk = k0 + kb * KB + r;
      const bool ok = gk < K && col < rows;
      const uint4 x = *(const uint4*)(g + (ok ? gk : 0) * ld + (ok ? col : 0));
      v[r] = ok ? x : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16* s) const {
    const int kb = XS ? threadIdx.x / NCB : threadIdx.x % NKB;
    const int cb = XS ? threadIdx.x % NCB : threadIdx.x / NKB;
    const uint32_t* w[KB];
#pragma unroll
    for (int r = 0; r < KB; ++r) w[r] = (const uint32_t*)&v[r];
#pragma unroll
    for (int d = 0; d < 4; ++d) {          // column pair (2d, 2d+1)
      if constexpr (KB == 8) {
        uint4 lo, hi;
        lo.x = lo_pair(w[0][d], w[1][d]); hi.x = hi_pair(w[0][d], w[1][d]);
        lo.y = lo_pair(w[2][d], w[3][d]); hi.y = hi_pair(w[2][d], w[3][d]);
        lo.z = lo_pair(w[4][d], w[5][d]); hi.z = hi_pair(w[4][d], w[5][d]);
        lo.w = lo_pair(w[6][d], w[7][d]); hi.w = hi_pair(w[6][d], w[7][d]);
        *(uint4*)(s + lds_at<XS>(cb * 8 + 2 * d, kb * 8)) = lo;
        *(uint4*)(s + lds_at<XS>(cb * 8 + 2 * d + 1, kb * 8)) = hi;
      } else {
        uint2 lo, hi;
        lo.x = lo_pair(w[0][d], w[1][d]); hi.x = hi_pair(w[0][d], w[1][d]);
        lo.y = lo_pair(w[2][d], w[3][d]); hi.y = hi_pair(w[2][d], w[3][d]);
        *(uint2*)(s + lds_at<XS>(cb * 8 + 2 * d, kb * 4)) = lo;
        *(uint2*)(s + lds_at<XS>(cb * 8 + 2 * d + 1, kb * 4)) = hi;
      }
    }
  }
};

template <bool TRANS, int R, int NT = 256, bool XS = false>
using Stage = typename std::conditional<TRANS, KColStage<R, NT, XS>, KRowStage<R, NT, XS>>::type;

// ------------------------------------------------------------ epilogue x4
// Four consecutive columns n..n+3 of row m (n % 4 == 0, N % 4 == 0).
// Epilogues that read memory (residual add: C; ReLU² backward: u; fp32
// accumulate: C) take what they read as `in`, loaded by epi_load, so a
// kernel can issue the loads of many fragments before the first one is used.
template <int EPI>
struct EpiIn {
  typedef uint2 type;       // 4 bf16
};
template <>
struct EpiIn<E_F32_ACC> {
  typedef f32x4_t type;
};
template <int EPI>
constexpr bool epi_reads() {
  return EPI == E_RESADD || EPI == E_DRELU2 || EPI == E_F32_ACC;
}

template <int EPI>
__device__ __forceinline__ typename EpiIn<EPI>::type epi_load(const void* Cv, const void* auxv,
                                                              int64_t i) {
  if constexpr (EPI == E_F32_ACC) return *(const f32x4_t*)((const float*)Cv + i);
  else if constexpr (EPI == E_DRELU2) return *(const uint2*)((const bf16*)auxv + i);
  else if constexpr (EPI == E_RESADD) return *(const uint2*)((const bf16*)Cv + i);
  else return uint2{0u, 0u};
}

template <int EPI>
__device__ __forceinline__ void epi4_in(void* Cv, void* auxv, int64_t i, f32x4_t a,
                                        typename EpiIn<EPI>::type in) {
  if constexpr (EPI == E_F32) {
    *(f32x4_t*)((float*)Cv + i) = a;
  } else if constexpr (EPI == E_F32_ACC) {
    *(f32x4_t*)((float*)Cv + i) = in + a;
  } else {
    bf16* C = (bf16*)Cv;
    float v[4] = {a[0], a[1], a[2], a[3]};
    if constexpr (EPI == E_RESADD) {
      v[0] += __uint_as_float(in.x << 16); v[1] += __uint_as_float(in.x & 0xFFFF0000u);
      v[2] += __uint_as_float(in.y << 16); v[3] += __uint_as_float(in.y & 0xFFFF0000u);
    } else if constexpr (EPI == E_DRELU2) {    // in: a = relu(u)^2, relu(u) = sqrt(a)
      v[0] *= 2.0f * __builtin_sqrtf(__uint_as_float(in.x << 16));
      v[1] *= 2.0f * __builtin_sqrtf(__uint_as_float(in.x & 0xFFFF0000u));
      v[2] *= 2.0f * __builtin_sqrtf(__uint_as_float(in.y << 16));
      v[3] *= 2.0f * __builtin_sqrtf(__uint_as_float(in.y & 0xFFFF0000u));
    }
    uint2 o;
    o.x = pack2bf(v[0], v[1]);
    o.y = pack2bf(v[2], v[3]);
    if constexpr (EPI == E_RELU2) {      // a = relu(u)^2 of u rounded to bf16
      float r0 = fmaxf(__uint_as_float(o.x << 16), 0.f), r1 = fmaxf(__uint_as_float(o.x & 0xFFFF0000u), 0.f);
      float r2 = fmaxf(__uint_as_float(o.y << 16), 0.f), r3 = fmaxf(__uint_as_float(o.y & 0xFFFF0000u), 0.f);
      o.x = pack2bf(r0 * r0, r1 * r1);
      o.y = pack2bf(r2 * r2, r3 * r3);
    }
    *(uint2*)(C + i) = o;
  }
}

template <int EPI>
__device__ __forceinline__ void epi4(void* Cv, void* auxv, int64_t ldc, int64_t m, int64_t n,
                                     f32x4_t a) {
  const int64_t i = m * ldc + n;
  epi4_in<EPI>(Cv, auxv, i, a, epi_load<EPI>(Cv, auxv, i));
}

// --------------------------------------------------------- one K-slice
// MFMAs of one 64-deep K-slice for a wave's (16 TMI) x (16 TNJ) sub-tile,
// software-pipelined: the B fragments of both 32-deep halves are read first,
// then the A fragments stream D ahead of the 4..8-MFMA group that consumes
// each one.  sched_barrier(0) pins that order: left alone, the scheduler
// sinks every LDS read next to its first use and the wave then waits out the
// full LDS latency before each group.
//
// D = 0 leaves the order to the compiler (better where the tile leaves no
// spare registers for the streamed fragments, as in the 4-wave kernels).
template <int TMI, int TNJ, bool XS, int D>
__device__ __forceinline__ void mma_slice(const bf16* As, const bf16* Bs, int wm, int wn, int lr,
                                          int lk, f32x4_t (&acc)[TMI][TNJ]) {
  if constexpr (D == 0) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[TMI], b[TNJ];
#pragma unroll
      for (int i = 0; i < TMI; ++i)
        a[i] = *(const bf16x8_t*)(As + lds_at<XS>(wm + 16 * i + lr, kk + lk));
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
        b[j] = *(const bf16x8_t*)(Bs + lds_at<XS>(wn + 16 * j + lr, kk + lk));
#pragma unroll
      for (int i = 0; i < TMI; ++i)
#pragma unroll
        for (int j = 0; j < TNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    return;
  }
  bf16x8_t b[2][TNJ];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < TNJ; ++j)
      b[h][j] = *(const bf16x8_t*)(Bs + lds_at<XS>(wn + 16 * j + lr, 32 * h + lk));
  constexpr int NA = 2 * TMI;
  constexpr int DD = D > 0 ? D : 1;
  bf16x8_t a[NA];
#pragma unroll
  for (int x = 0; x < DD; ++x)
    a[x] = *(const bf16x8_t*)(As + lds_at<XS>(wm + 16 * (x % TMI) + lr, 32 * (x / TMI) + lk));
#pragma unroll
  for (int x = 0; x < NA; ++x) {
    if (x + DD < NA) {
      const int y = x + DD;
      a[y] = *(const bf16x8_t*)(As + lds_at<XS>(wm + 16 * (y % TMI) + lr, 32 * (y / TMI) + lk));
    }
    __builtin_amdgcn_sched_barrier(0);
    const int i = x % TMI, h = x / TMI;
#pragma unroll
    for (int j = 0; j < TNJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[h][j], a[x], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------ kernel
struct TileMap {
  int tiles_m, tiles_n, splits;
  int64_t k_per_split;     // multiple of BK
  // batched products: element strides between the batch's A, B and C
  // matrices; when batch > 1 the batch index comes from a 1-D grid over
  // batch x tiles numbered like a product's tiles (each XCD a contiguous
  // run, so the tiles of one matrix share at most two L2s), else from
  // blockIdx.y
  int64_t bs_a = 0, bs_b = 0, bs_c = 0;
  int batch = 0;
  // E_CE only: per-(row, column tile) stats, target logits, token rows
  float* ce_stats = nullptr;
  float* ce_zt = nullptr;
  const int32_t* ce_tok = nullptr;
  int ce_T = 1;
  int ce_direct = 0;
  // E_CEB only: per-row lse, and the gradient's scale (1 / tokens)
  const float* ce_lse = nullptr;
  float ce_scale = 0.f;
  // E_QKNORM only
  const float2* qk_cs = nullptr;
  float* qk_rq = nullptr;
  float* qk_rk = nullptr;
  int qk_T = 1, qk_H = 0, qk_Hkv = 0;
  float qk_eps = 0.f;
  // E_QKNORM, value-embedding layers: v += g E[token], g = 3 sigmoid(h[:, :C] wg^T)
  const int32_t* ve_tok = nullptr;
  const bf16* ve_h = nullptr;
  const bf16* ve_wg = nullptr;
  const bf16* ve_E = nullptr;
  float* ve_g = nullptr;
  int ve_D = 0, ve_C = 0;
  // tile order inside one K split: 0 = column-major groups of 8 tile rows;
  // 1 = row by row (tile_m slow), 2 = column by column (tile_n slow)
  int order = 0;
};

// (tile_m, tile_n) of tile t of a split, in the order the plan chose.  The
// blocks of one split are dealt to consecutive XCDs; with split K the run of
// a split's tiles usually crosses an XCD boundary, and each XCD then reads
// every panel its part of the run touches.  Row by row (or column by
// column) order cuts the run across the larger operand's panels only once,
// so only the smaller operand's panels are read by both XCDs.
__device__ __forceinline__ void tile_of(const TileMap& tm, int t, int& tile_m, int& tile_n) {
  if (tm.order == 1) {
    tile_m = t / tm.tiles_n;
    tile_n = t % tm.tiles_n;
  } else if (tm.order == 2) {
    tile_n = t / tm.tiles_m;
    tile_m = t % tm.tiles_m;
  } else {
    constexpr int GM = 8;
    const int group = t / (GM * tm.tiles_n);
    const int first_m = group * GM;
    const int gsize = min(tm.tiles_m - first_m, GM);
    tile_m = first_m + (t % (GM * tm.tiles_n)) % gsize;
    tile_n = (t % (GM * tm.tiles_n)) / gsize;
  }
}

template <int BM, int BN, bool TA, bool TB, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(int64_t M, int64_t N, int64_t K,
                                                      const bf16* __restrict__ A, int64_t lda,
                                                      const bf16* __restrict__ B, int64_t ldb,
                                                      void* C, int64_t ldc, void* aux,
                                                      TileMap tm, float* partial) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TMI = WM / 16, TNJ = WN / 16;
  __shared__ __attribute__((aligned(16))) bf16 As[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[BN * LDK];
  // ---- which tile: XCD-contiguous numbering (of (matrix, tile) pairs when
  // batched), then grouped column-major
  const int nb1 = tm.tiles_m * tm.tiles_n * tm.splits;
  const int nb = tm.batch > 1 ? nb1 * tm.batch : nb1;
  const int per_xcd = (nb + 7) / 8;
  int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= nb) return;
  int bz = (int)blockIdx.y;
  if (tm.batch > 1) {
    bz = logical / nb1;
    logical -= bz * nb1;
  }
  if (bz) {
    constexpr int ce = (EPI == E_F32 || EPI == E_F32_ACC) ? 4 : 2;
    A += bz * tm.bs_a;
    B += bz * tm.bs_b;
    C = (char*)C + bz * tm.bs_c * ce;
  }
  const int ntile = tm.tiles_m * tm.tiles_n;
  const int split = logical / ntile;
  const int t = logical % ntile;
  int tile_m, tile_n;
  tile_of(tm, t, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int64_t kbeg = (int64_t)split * tm.k_per_split;
  const int64_t kend = min(K, kbeg + tm.k_per_split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  f32x4_t acc[TMI][TNJ];
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr bool XS = TA && TB;
  Stage<TA, BM, 256, XS> sa;
  Stage<TB, BN, 256, XS> sb;
  sa.load(A, lda, m0, M, kbeg, kend);
  sb.load(B, ldb, n0, N, kbeg, kend);
  sa.store(As);
  sb.store(Bs);
  __syncthreads();

  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) {
      sa.load(A, lda, m0, M, k0 + BK, kend);
      sb.load(B, ldb, n0, N, k0 + BK, kend);
    }
    mma_slice<TMI, TNJ, XS, 0>(As, Bs, wm, wn, lr, lk, acc);
    __syncthreads();
    if (more) {
      sa.store(As);
      sb.store(Bs);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows m = .. + lr, columns n = .. + 4*(lane>>4) + 0..3
  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const int64_t m = m0 + wm + 16 * i + lr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TNJ; ++j) {
      const int64_t n = n0 + wn + 16 * j + cq;
      if (n >= N) continue;
      if (partial) {
        *(f32x4_t*)(partial + ((int64_t)split * M + m) * N + n) = acc[i][j];
      } else {
        epi4<EPI>(C, aux, ldc, m, n, acc[i][j]);
      }
    }
  }
}

// Large-tile variant: 256 x 256 block tile, 8 waves (2 x 4, each 128 x 64),
// two LDS stages.  The next K-slice is fetched into registers while the
// current stage is consumed and written into the other stage afterwards, so
// one barrier per K-slice suffices (the barrier that publishes stage s+1 also
// retires every read of stage s before it is overwritten).  One block per CU
// (144 KB of LDS), two waves per SIMD.
template <bool TA, bool TB, int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_mfma_db(int64_t M, int64_t N, int64_t K,
                                                         const bf16* __restrict__ A, int64_t lda,
                                                         const bf16* __restrict__ B, int64_t ldb,
                                                         void* C, int64_t ldc, void* aux,
                                                         TileMap tm, float* partial) {
  constexpr int BM = 256, BN = 256, NT = 512;
  constexpr int WM = 128, WN = 64;
  constexpr int TMI = WM / 16, TNJ = WN / 16;
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * (BM + BN) * LDK];
  bf16* As0 = lds;
  bf16* Bs0 = lds + BM * LDK;
  bf16* As1 = lds + (BM + BN) * LDK;
  bf16* Bs1 = lds + (2 * BM + BN) * LDK;

  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int per_xcd = (nb + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= nb) return;
  const int ntile = tm.tiles_m * tm.tiles_n;
  const int split = logical / ntile;
  const int t = logical % ntile;
  int tile_m, tile_n;
  tile_of(tm, t, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int64_t kbeg = (int64_t)split * tm.k_per_split;
  const int64_t kend = min(K, kbeg + tm.k_per_split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = (wave >> 2) * WM, wn = (wave & 3) * WN;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  f32x4_t acc[TMI][TNJ];
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stage<TA, BM, NT> sa;
  Stage<TB, BN, NT> sb;
  sa.load(A, lda, m0, M, kbeg, kend);
  sb.load(B, ldb, n0, N, kbeg, kend);
  sa.store(As0);
  sb.store(Bs0);
  __syncthreads();

  int stage = 0;
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) {
      sa.load(A, lda, m0, M, k0 + BK, kend);
      sb.load(B, ldb, n0, N, k0 + BK, kend);
    }
    const bf16* As = stage ? As1 : As0;
    const bf16* Bs = stage ? Bs1 : Bs0;
    mma_slice<TMI, TNJ, false, 2>(As, Bs, wm, wn, lr, lk, acc);
    if (more) {
      sa.store(stage ? As0 : As1);
      sb.store(stage ? Bs0 : Bs1);
    }
    __syncthreads();
    stage ^= 1;
  }

  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const int64_t m = m0 + wm + 16 * i + lr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TNJ; ++j) {
      const int64_t n = n0 + wn + 16 * j + cq;
      if (n >= N) continue;
      if (partial) {
        *(f32x4_t*)(partial + ((int64_t)split * M + m) * N + n) = acc[i][j];
      } else {
        epi4<EPI>(C, aux, ldc, m, n, acc[i][j]);
      }
    }
  }
}

// ------------------------------------------------- direct-to-LDS variant
// 8 waves (4 x 2, each (BM/4) x (BN/2)), LDS stages filled straight from
// global memory by buffer_load_dwordx4 ... lds: every load instruction moves
// one contiguous 1 KB LDS block (lane i -> bytes 16i..16i+15), so the layout
// is chosen through which global 16-byte chunk each lane fetches.  No
// staging registers and no LDS store instructions; A is fetched two K-slices
// ahead (a ring of three stages), B one slice ahead (a ring of two), so the
// loads of slices s+1 and s+2 stay in flight while slice s is multiplied.
//
// K-contiguous operand: LDS rows of 64 k (128 B, no padding), 16-byte chunk c
// of row r stored at position c ^ ((r >> 1) & 7); a fragment read (16 rows,
// one chunk) then touches 16 distinct 16-byte bank slots.
// MN-contiguous operand: LDS rows are k (R elements each, as in memory), and
// a fragment is gathered with two ds_read_b64_tr_b16: in each 16-lane group,
// lane s points at 4 elements (row k0 + s/4, columns 4(s%4)..) and receives
// the 4 k-values of column s (its MFMA operand layout).  Chunks are XOR-
// swizzled per k row so the 8 rows one read instruction touches per 32 lanes
// fall in distinct 32-byte bank slots.
//
// K must be a multiple of 64 (no zero fill: rows past M or N are clamped to
// valid memory and their results dropped).

__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }

// chunk swizzle of k-row `k` in an MN-contiguous stage of R columns
template <int R>
__device__ __forceinline__ int swz_mn(int k) {
  if constexpr (R == 192) return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));
  else return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
}

// Buffer loads straight into LDS.  The descriptor of an operand starts at
// the tile's first row (K-contiguous) or column (MN-contiguous) and ends at
// the end of the matrix, so lanes past the last row or k read zeros; columns
// past N alias into the next row and only feed results that are dropped.
// One per-lane byte offset per operand: the NB load instructions of a wave
// differ by a uniform step (64 rows, or 4096 / R k-rows, with the same
// swizzle), added to it per instruction (the whole offset stays in the
// vector operand, which is what the range check sees).
template <int R, bool TRANS>
struct DmaPlan {
  static constexpr int NB = R / 64;                        // load instructions per wave
  static constexpr int STEP_ROWS = TRANS ? 4096 / R : 64;  // rows (k or MN) between them
  // an MN-contiguous stage of 192 columns has 384-byte rows, which 1 KB load
  // blocks do not tile evenly: one offset per load instruction there
  static constexpr bool PER_LOAD = TRANS && R == 192;
  static constexpr int NV = PER_LOAD ? NB : 1;
  static_assert(!TRANS || R == 128 || R == 192 || R == 256, "MN-contiguous stage width");
  i32x4_t rsrc;
  uint32_t voff[NV];
  int64_t ld;
  // g: operand base; r0: first MN index of the tile; rows: M or N; K rows
  __device__ __forceinline__ void init(const bf16* g, int64_t ld_, int64_t r0, int64_t rows,
                                       int64_t K, int wave, int lane) {
    ld = ld_;
    if constexpr (!TRANS) {
      const int o = 1024 * wave + 16 * lane;    // byte offset of this lane in block `wave`
      const int row = o >> 7, p = (o >> 4) & 7;
      rsrc = make_rsrc(g + r0 * ld, (rows - r0) * ld * 2);
      voff[0] = (uint32_t)(row * ld * 2 + 16 * (p ^ swz_k(row)));
    } else {
      rsrc = make_rsrc(g + r0, (K * ld - r0) * 2);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int o = 1024 * (wave + 8 * i) + 16 * lane;
        const int krow = o / (2 * R), p = (o % (2 * R)) >> 4;
        voff[i] = (uint32_t)(krow * ld * 2 + 16 * (p ^ swz_mn<R>(krow)));
      }
    }
  }
  __device__ __forceinline__ void issue(int64_t k0, bf16* stage, int wave) const {
    const uint32_t kofs = (uint32_t)(TRANS ? k0 * ld * 2 : k0 * 2);
    const uint32_t step = (uint32_t)(STEP_ROWS * ld * 2);
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)stage + 1024u * (uint32_t)wave);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      dma16(rsrc, base + 8192u * i, (PER_LOAD ? voff[i] : voff[0] + i * step) + kofs);
  }
};

// fragment (16 rows of the MN index from `base`, k = kk + 8g .. +7) of a
// stage operand
template <int R, bool TRANS>
__device__ __forceinline__ bf16x8_t frag(const bf16* st, int base, int kk, int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  if constexpr (!TRANS) {
    const int row = base + l16, c = (kk >> 3) + g;
    return *(const bf16x8_t*)(st + row * 64 + 8 * (c ^ swz_k(row)));
  } else {
    const int n = base + 4 * (l16 & 3), c = n >> 3;
    v4s_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = kk + 8 * g + 4 * hh + (l16 >> 2);
      const bf16* p = st + k * R + 8 * (c ^ swz_mn<R>(k)) + (n & 7);
      h[hh] = tr16(p);
    }
    typedef short v8s_t __attribute__((ext_vector_type(8)));
    v8s_t v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

// Epilogue of one wave's TMI x TNJ accumulator fragments: lane (g, lr)
// holds rows r0 + 16 i + lr, columns c0 + 16 j + 4 g .. + 3.  With P (split
// K) the fp32 partial tile goes there; otherwise EPI applies.
template <int EPI, int TMI, int TNJ>
__device__ __forceinline__ void store_tiles(const f32x4_t (&acc)[TMI][TNJ], int64_t M, int64_t N,
                                            int64_t r0, int64_t c0, int lane, void* C,
                                            int64_t ldc, void* aux, float* P) {
  const int cq = (lane >> 4) * 4, lr = lane & 15;
  if (P) {
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int64_t m = r0 + 16 * i + lr;
#pragma unroll
      for (int j = 0; j < TNJ; ++j) {
        const int64_t n = c0 + 16 * j + cq;
        if (m < M && n < N) *(f32x4_t*)(P + m * N + n) = acc[i][j];
      }
    }
    return;
  }
  // per pair of 16-row groups (one group for fp32 inputs): every load of
  // the groups first, then the stores (one memory latency per batch instead
  // of one per fragment; the MFMA operand registers are free by now)
  constexpr int GB = (EPI == E_F32_ACC || TMI % 2) ? 1 : 2;
  if constexpr (EPI == E_F32_ACC) {
    // read-add-write one fragment at a time (hoisting these loads above the
    // main loop costs the accumulators their registers)
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int64_t m = r0 + 16 * i + lr;
#pragma unroll
      for (int j = 0; j < TNJ; ++j) {
        const int64_t n = c0 + 16 * j + cq;
        if (m < M && n < N) {
          f32x4_t* p = (f32x4_t*)((float*)C + m * ldc + n);
          f32x4_t v = __builtin_nontemporal_load(p);
          asm volatile("" : "+v"(v));
          *p = v + acc[i][j];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i0 = 0; i0 < TMI; i0 += GB) {
    typename EpiIn<EPI>::type in[GB][TNJ];
    if constexpr (epi_reads<EPI>()) {
#pragma unroll
      for (int gi = 0; gi < GB; ++gi) {
        const int64_t m = r0 + 16 * (i0 + gi) + lr;
#pragma unroll
        for (int j = 0; j < TNJ; ++j) {
          const int64_t n = c0 + 16 * j + cq;
          if (m < M && n < N) in[gi][j] = epi_load<EPI>(C, aux, m * ldc + n);
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < GB; ++gi) {
      const int64_t m = r0 + 16 * (i0 + gi) + lr;
#pragma unroll
      for (int j = 0; j < TNJ; ++j) {
        const int64_t n = c0 + 16 * j + cq;
        if (m < M && n < N) epi4_in<EPI>(C, aux, m * ldc + n, acc[i0 + gi][j], in[gi][j]);
      }
    }
  }
}

template <int BM, int BN, bool TA, bool TB, int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_dma(int64_t M, int64_t N, int64_t K,
                                                     const bf16* __restrict__ A, int64_t lda,
                                                     const bf16* __restrict__ B, int64_t ldb,
                                                     void* C, int64_t ldc, void* aux,
                                                     TileMap tm, float* partial) {
  constexpr int WM = BM / 4, WN = BN / 2;
  constexpr int TMI = WM / 16, TNJ = WN / 16;
  // LDS: a ring of three A tiles and two B tiles (below); E_CEB also keeps
  // the tile's 256 rows' lse and two slots of their vocabulary-tile maxima
  constexpr int SX = EPI == E_CEB ? 3 * 256 * 2 : 0;
  __shared__ __attribute__((aligned(1024))) bf16 lds[(3 * BM + 2 * BN) * 64 + SX];
  const int nb1 = tm.tiles_m * tm.tiles_n * tm.splits;
  const int nb = tm.batch > 1 ? nb1 * tm.batch : nb1;
  const int per_xcd = (nb + 7) / 8;
  int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= nb) return;
  int bz = (int)blockIdx.y;
  if (tm.batch > 1) {
    bz = logical / nb1;
    logical -= bz * nb1;
  }
  if (bz) {
    constexpr int ce = (EPI == E_F32 || EPI == E_F32_ACC) ? 4 : 2;
    A += bz * tm.bs_a;
    B += bz * tm.bs_b;
    C = (char*)C + bz * tm.bs_c * ce;
  }
  const int ntile = tm.tiles_m * tm.tiles_n;
  const int split = logical / ntile;
  const int t = logical % ntile;
  int tile_m, tile_n;
  tile_of(tm, t, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int64_t kbeg = (int64_t)split * tm.k_per_split;
  const int64_t kend = min(K, kbeg + tm.k_per_split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  DmaPlan<BM, TA> pa;
  DmaPlan<BN, TB> pb;
  pa.init(A, lda, m0, M, K, wave, lane);
  pb.init(B, ldb, n0, N, K, wave, lane);

  f32x4_t acc[TMI][TNJ];
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // E_CEB (A = e = exp(logit - m_t), K = the vocabulary): the accumulator
  // of each row is kept in units of exp(m'_t) for the 256-column tile t
  // being summed, m'_t = max(m_t, lse - 40), and multiplied by exp(m'_(t-1)
  // - m'_t) when a tile starts.  Every m' lies in [lse - 40, lse], so the
  // factors stay within e^(+-40); a tile whose max is more than 40 below
  // lse counts as if it were 40 below, a change far under bf16 resolution
  // (its true weight is below e^-40).  The factors of a tile are applied
  // after the carried products of the previous tile's last slice and
  // before the tile's own first products.  The lse of the block's rows and
  // each tile's maxima reach LDS by buffer loads (waves 0-3, one row a
  // lane) issued ahead of a slice's operand loads, so the per-slice waits
  // cover them and no other load is in flight in the main loop; the maxima
  // of tile t + 1 are fetched when tile t starts.
  float cb_lse[TMI], cb_m[TMI];
  const int ntv = (int)(K >> 8);
  // floats [0, 256): lse; [256, 512) and [512, 768): maxima of the even and
  // the odd tiles
  float* const cb_lds = (float*)(lds + (3 * BM + 2 * BN) * 64);
  // descriptors and the wave test are uniform (scalar registers, branch)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const i32x4_t cb_rs = make_rsrc(EPI == E_CEB ? tm.ce_stats : nullptr, M * ntv * 8);
  const uint32_t cb_off = (uint32_t)(min(m0 + 64 * (wave & 3) + lane, M - 1) * ntv * 8);
  auto cb_issue = [&](int t) {             // maxima of tile t
    if (wv < 4) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_void_t*)(cb_lds + 256 * (1 + (t & 1)) + 64 * wv));
      dma4(cb_rs, dst, cb_off + 8u * (uint32_t)t);
    }
  };
  if constexpr (EPI == E_CEB) {
    const i32x4_t cb_rl = make_rsrc(tm.ce_lse, M * 4);
    if (wv < 4) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_void_t*)(cb_lds + 64 * wv));
      dma4(cb_rl, dst, (uint32_t)(min(m0 + 64 * wv + lane, M - 1) * 4));
    }
    cb_issue(0);
  }

  const int nsl = (int)((kend - kbeg) / BK);
  int it = 0;
  // A ring of three, B ring of two: A (the activations or gradients, the
  // operand that streams from HBM) is fetched two slices ahead, B one.
  // Per slice: wait until only A(s + 1) is in flight (loads land in issue
  // order and A(s + 1) went out after B(s)), barrier (every wave is done
  // with slice s - 1, whose A and B stages the next loads reuse), issue
  // B(s + 1) then A(s + 2), multiply slice s.
  bf16* const ra = lds;                    // A stages: ra + j BM 64
  bf16* const rb = lds + 3 * BM * 64;      // B stages: rb + j BN 64
  constexpr int NA = DmaPlan<BM, TA>::NB;  // A loads per wave and slice
  pa.issue(kbeg, ra, wave);
  pb.issue(kbeg, rb, wave);
  if (nsl > 1) pa.issue(kbeg + BK, ra + BM * 64, wave);
  // The second half slice's products are carried over the next barrier:
  // its fragments are read before it, and its MFMAs cover the latency of
  // the next slice's first reads (every wave reads at the same moment,
  // right after the barrier).
  auto rd = [&](bf16x8_t (&a)[TMI], bf16x8_t (&b)[TNJ], const bf16* As, const bf16* Bs,
                int kk) {
#pragma unroll
    for (int j = 0; j < TNJ; ++j) b[j] = frag<BN, TB>(Bs, wn + 16 * j, kk, lane);
#pragma unroll
    for (int i = 0; i < TMI; ++i) a[i] = frag<BM, TA>(As, wm + 16 * i, kk, lane);
  };
  auto mm = [&](const bf16x8_t (&a)[TMI], const bf16x8_t (&b)[TNJ]) {
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  bf16x8_t fa[TMI], fb[TNJ], ga[TMI], gb[TNJ];   // first / second half slice
  int sa = 0, sb = 0;                      // stages of slice `it`
  for (; it < nsl; ++it) {
    if (it + 1 < nsl) dma_wait_n<NA>();
    else dma_wait();
    __syncthreads();
    if constexpr (EPI == E_CEB)
      if ((it & 3) == 0 && (it >> 2) + 1 < ntv) cb_issue((it >> 2) + 1);
    const int sa2 = sa == 0 ? 2 : sa - 1;  // (it + 2) % 3
    if (it + 1 < nsl) pb.issue(kbeg + (int64_t)(it + 1) * BK, rb + (sb ^ 1) * BN * 64, wave);
    if (it + 2 < nsl) pa.issue(kbeg + (int64_t)(it + 2) * BK, ra + sa2 * BM * 64, wave);
    const bf16* As = ra + sa * BM * 64;
    const bf16* Bs = rb + sb * BN * 64;
    rd(fa, fb, As, Bs, 0);
    if (it > 0) mm(ga, gb);                // slice it - 1, second half
    if constexpr (EPI == E_CEB) {
      if ((it & 3) == 0) {                 // a 256-wide vocabulary tile starts
        const int t = it >> 2;
        const float* mx = cb_lds + 256 * (1 + (t & 1)) + wm + (lane & 15);
        if (t == 0) {
#pragma unroll
          for (int i = 0; i < TMI; ++i) cb_lse[i] = cb_lds[wm + 16 * i + (lane & 15)];
        }
#pragma unroll
        for (int i = 0; i < TMI; ++i) {
          const float mt = fmaxf(mx[16 * i], cb_lse[i] - 40.f);
          if (t > 0) {                       // the accumulator is zero at t = 0
            const float f = __builtin_amdgcn_exp2f((cb_m[i] - mt) * 1.4426950408889634f);
#pragma unroll
            for (int j = 0; j < TNJ; ++j) acc[i][j] *= f;
          }
          cb_m[i] = mt;
        }
      }
    }
    mm(fa, fb);
    rd(ga, gb, As, Bs, 32);
    sa = sa == 2 ? 0 : sa + 1;
    sb ^= 1;
  }
  if (nsl > 0) mm(ga, gb);
  const int cq = (lane >> 4) * 4, lr = lane & 15;
  if constexpr (EPI == E_CE) {
    // Fused lm_head + cross-entropy, first half (the tile is 256 x 256 and
    // every column is a valid vocabulary entry): per row of the tile, the
    // max m of its 256 logits and s = sum exp(logit - m) in fp32, e = exp(
    // logit - m) as bf16 (when C is given), and the target's logit.  The
    // two waves sharing a row combine through LDS (the stages are free).
    const int ntn = tm.tiles_n;
    int tg[TMI];
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int64_t m = m0 + wm + 16 * i + lr;
      tg[i] = m >= M ? -1
              : tm.ce_direct ? tm.ce_tok[m]
                             : tm.ce_tok[(m / tm.ce_T) * (tm.ce_T + 1) + m % tm.ce_T + 1];
    }
    __syncthreads();
    float* red = (float*)lds;              // [0, 512): maxima, [512, 1024): sums
    float mx[TMI];
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      // the one lane holding the row's target column stores its logit
      const int lc = tg[i] - (int)n0 - wn;           // column within this wave's 128
      if (lc >= 0 && lc < WN && ((lc >> 2) & 3) == (lane >> 4)) {
        const int jj = lc >> 4, rr = lc & 3;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < TNJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) v = (j == jj && r == rr) ? acc[i][j][r] : v;
        tm.ce_zt[m0 + wm + 16 * i + lr] = v;
      }
      float v = -INFINITY;
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v = fmaxf(v, acc[i][j][r]);
      v = fmaxf(v, __shfl_xor(v, 16, 64));
      v = fmaxf(v, __shfl_xor(v, 32, 64));
      if (lane < 16) red[(wave & 1) * 256 + wm + 16 * i + lr] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int rr = wm + 16 * i + lr;
      mx[i] = fmaxf(red[rr], red[256 + rr]);
      const float mxl = mx[i] * 1.4426950408889634f;
      float sacc = 0.f;
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], 1.4426950408889634f, -mxl));
          acc[i][j][r] = e;
          sacc += e;
        }
      sacc += __shfl_xor(sacc, 16, 64);
      sacc += __shfl_xor(sacc, 32, 64);
      if (lane < 16) red[512 + (wave & 1) * 256 + rr] = sacc;
    }
    __syncthreads();
    if ((wave & 1) == 0 && lane < 16) {
#pragma unroll
      for (int i = 0; i < TMI; ++i) {
        const int rr = wm + 16 * i + lr;
        const int64_t m = m0 + rr;
        if (m < M)
          *(float2*)(tm.ce_stats + 2 * (m * ntn + tile_n)) =
              make_float2(mx[i], red[512 + rr] + red[768 + rr]);
      }
    }
    if (C) {
#pragma unroll
      for (int i = 0; i < TMI; ++i) {
        const int64_t m = m0 + wm + 16 * i + lr;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < TNJ; ++j) {
          const int64_t n = n0 + wn + 16 * j + cq;
          uint2 u;
          u.x = pack2bf(acc[i][j][0], acc[i][j][1]);
          u.y = pack2bf(acc[i][j][2], acc[i][j][3]);
          *(uint2*)((uint16_t*)C + m * ldc + n) = u;
        }
      }
    }
    return;
  }
  if constexpr (EPI == E_CEB) {
    // dh = (softmax - onehot(target)) grad_scale times Wlm: the accumulator
    // (units exp(m'_last)) times exp(m'_last - lse) grad_scale, minus the
    // target's row of Wlm (B) times grad_scale
    const float sc = tm.ce_scale;
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int64_t m = m0 + wm + 16 * i + lr;
      if (m >= M) continue;
      const float f = __builtin_amdgcn_exp2f((cb_m[i] - cb_lse[i]) * 1.4426950408889634f) * sc;
      const int tg = tm.ce_direct ? tm.ce_tok[m]
                                  : tm.ce_tok[(m / tm.ce_T) * (tm.ce_T + 1) + m % tm.ce_T + 1];
      const bf16* wrow = B + (int64_t)tg * ldb;
#pragma unroll
      for (int j = 0; j < TNJ; ++j) {
        const int64_t n = n0 + wn + 16 * j + cq;
        if (n >= N) continue;
        const uint2 wv = *(const uint2*)(wrow + n);
        uint2 o;
        o.x = pack2bf(fmaf(acc[i][j][0], f, -sc * __uint_as_float(wv.x << 16)),
                      fmaf(acc[i][j][1], f, -sc * __uint_as_float(wv.x & 0xFFFF0000u)));
        o.y = pack2bf(fmaf(acc[i][j][2], f, -sc * __uint_as_float(wv.y << 16)),
                      fmaf(acc[i][j][3], f, -sc * __uint_as_float(wv.y & 0xFFFF0000u)));
        *(uint2*)((bf16*)C + m * ldc + n) = o;
      }
    }
    return;
  }
  if constexpr (EPI == E_QKNORM) {
    // RoPE then RMS-norm per q / k head: the wave's 128 columns are one head
    // (256-wide tiles, head_dim 128); lane (g, lr) holds dims 16 j + 4 g + r,
    // so the rotation pairs (d, d + 64) are fragments j and j + 4 of one lane
    // and a row's sum of squares needs two shuffles.  u rounded to bf16
    // first, as the stored product would be.
    static_assert(WN == 128, "one head per wave");
    const int head = (int)((n0 + wn) >> 7);
    const int H = tm.qk_H, Hkv = tm.qk_Hkv;
#pragma unroll
    for (int i = 0; i < TMI; ++i) {
      const int64_t m = m0 + wm + 16 * i + lr;
      float x[TNJ][4];
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[j][r] = bf2f(f2bf(acc[i][j][r]));
      if (head < H + Hkv) {
        const int t = (int)((m < M ? m : 0) % tm.qk_T);
        const float2* cst = tm.qk_cs + (int64_t)t * 64;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < TNJ / 2; ++j) {
          const float4* c4 = (const float4*)(cst + 16 * j + cq);
          const float4 ca = c4[0], cb = c4[1];
          const float c[4] = {ca.x, ca.z, cb.x, cb.z}, sn[4] = {ca.y, ca.w, cb.y, cb.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x1 = x[j][r], x2 = x[j + 4][r];
            const float y1 = x1 * c[r] - x2 * sn[r], y2 = x1 * sn[r] + x2 * c[r];
            x[j][r] = y1;
            x[j + 4][r] = y2;
            ss += y1 * y1 + y2 * y2;
          }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float rr = 1.0f / sqrtf(ss / 128.0f + tm.qk_eps);
#pragma unroll
        for (int j = 0; j < TNJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[j][r] *= rr;
        if ((lane >> 4) == 0 && m < M) {
          if (head < H) tm.qk_rq[m * H + head] = rr;
          else tm.qk_rk[m * Hkv + (head - H)] = rr;
        }
      } else if (tm.ve_E && head < H + 2 * Hkv) {
        // value embedding of KV head hv: the gate is a C-long dot product
        // of the row's normalised input with wg[hv] (the row's four lanes
        // take every fourth channel), then v = v + g E[token] in fp32, one
        // rounding
        const int hv = head - H - Hkv;
        const int64_t mm = m < M ? m : 0;
        float ga = 0.f;
        if (tm.ve_C % 8 == 0) {
          // 8 consecutive channels per lane and step (16-byte loads)
          for (int c = 8 * (lane >> 4); c < tm.ve_C; c += 32) {
            const uint4 hv8 = *(const uint4*)(tm.ve_h + mm * tm.ve_D + c);
            const uint4 wv8 = *(const uint4*)(tm.ve_wg + (int64_t)hv * tm.ve_C + c);
            const uint32_t* hw = (const uint32_t*)&hv8;
            const uint32_t* ww = (const uint32_t*)&wv8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ga = fmaf(__uint_as_float(hw[e] << 16), __uint_as_float(ww[e] << 16), ga);
              ga = fmaf(__uint_as_float(hw[e] & 0xFFFF0000u), __uint_as_float(ww[e] & 0xFFFF0000u), ga);
            }
          }
        } else {
          for (int c = lane >> 4; c < tm.ve_C; c += 4)
            ga = fmaf(bf2f(tm.ve_h[mm * tm.ve_D + c]), bf2f(tm.ve_wg[(int64_t)hv * tm.ve_C + c]), ga);
        }
        ga += __shfl_xor(ga, 16, 64);
        ga += __shfl_xor(ga, 32, 64);
        const float gv = 3.0f / (1.0f + expf(-ga));
        if ((lane >> 4) == 0 && m < M) tm.ve_g[m * Hkv + hv] = gv;
        const int id = tm.ve_tok[(mm / tm.qk_T) * (tm.qk_T + 1) + mm % tm.qk_T];
        const bf16* er = tm.ve_E + (int64_t)id * (Hkv * 128) + hv * 128 + cq;
#pragma unroll
        for (int j = 0; j < TNJ; ++j) {
          const uint2 e = *(const uint2*)(er + 16 * j);
          x[j][0] = fmaf(gv, __uint_as_float(e.x << 16), x[j][0]);
          x[j][1] = fmaf(gv, __uint_as_float(e.x & 0xFFFF0000u), x[j][1]);
          x[j][2] = fmaf(gv, __uint_as_float(e.y << 16), x[j][2]);
          x[j][3] = fmaf(gv, __uint_as_float(e.y & 0xFFFF0000u), x[j][3]);
        }
      }
      if (m < M) {
#pragma unroll
        for (int j = 0; j < TNJ; ++j) {
          const int64_t n = n0 + wn + 16 * j + cq;
          if (n < N) {
            uint2 o;
            o.x = pack2bf(x[j][0], x[j][1]);
            o.y = pack2bf(x[j][2], x[j][3]);
            *(uint2*)((bf16*)C + m * ldc + n) = o;
          }
        }
      }
    }
    return;
  }
  store_tiles<EPI>(acc, M, N, m0 + wm, n0 + wn, lane, C, ldc, aux,
                   partial ? partial + (int64_t)split * M * N : nullptr);
}

// --------------------------------------------------------------- FP8
// C = (A B^T) * a_inv[0] * b_inv[0] for 8-bit float operands, both K-
// contiguous (A [M, K], B [N, K]; the transposed products of a layer's
// backward take transposed copies, which the cast kernel writes).  Same
// structure as k_gemm_dma: 256 x BN tiles, buffer loads straight into LDS,
// two stages.  A stage holds 128 k per row -- 128 bytes, the bf16 stages'
// row length -- so the bf16 operand plans and fragment reads serve
// unchanged, with the byte matrices viewed as 2-byte units.  Each stage is
// one v_mfma_f32_16x16x128_f8f6f4 per fragment pair: a lane brings 32 bytes
// of its row (the 16-byte chunks g and g + 4, the same k positions for
// both operands, so their products pair up whatever order the instruction
// sums them in).  FA / FB: 0 = e4m3, 1 = e5m2.  Twice the bf16 rate per
// instruction and half the bytes per k.  The stages form the bf16 kernel's
// rings: three A stages fetched two slices ahead, two B stages one ahead.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int R>
__device__ __forceinline__ i32x8_t frag_f8(const bf16* st, int base, int lane) {
  const bf16x8_t lo = frag<R, false>(st, base, 0, lane);
  const bf16x8_t hi = frag<R, false>(st, base, 32, lane);
  typedef short v8s_t __attribute__((ext_vector_type(8)));
  typedef short v16s_t __attribute__((ext_vector_type(16)));
  const v16s_t v = __builtin_shufflevector(__builtin_bit_cast(v8s_t, lo),
                                           __builtin_bit_cast(v8s_t, hi), 0, 1, 2, 3, 4, 5, 6,
                                           7, 8, 9, 10, 11, 12, 13, 14, 15);
  return __builtin_bit_cast(i32x8_t, v);
}

template <int BN, int FA, int FB, int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8(int64_t M, int64_t N, int64_t Ku,
                                                     const bf16* __restrict__ A, int64_t ldau,
                                                     const bf16* __restrict__ B, int64_t ldbu,
                                                     const float* __restrict__ a_inv,
                                                     const float* __restrict__ b_inv, void* C,
                                                     int64_t ldc, TileMap tm, float* partial) {
  // Ku, ldau, ldbu, tm.k_per_split: in 2-byte units (2 fp8 values each)
  constexpr int BM = 256;
  constexpr int WM = BM / 4, WN = BN / 2;
  constexpr int TMI = WM / 16, TNJ = WN / 16;
  __shared__ __attribute__((aligned(1024))) bf16 lds[(3 * BM + 2 * BN) * 64];

  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int per_xcd = (nb + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= nb) return;
  const int ntile = tm.tiles_m * tm.tiles_n;
  const int split = logical / ntile;
  const int t = logical % ntile;
  int tile_m, tile_n;
  tile_of(tm, t, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int64_t kbeg = (int64_t)split * tm.k_per_split;
  const int64_t kend = min(Ku, kbeg + tm.k_per_split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  DmaPlan<BM, false> pa;
  DmaPlan<BN, false> pb;
  pa.init(A, ldau, m0, M, Ku, wave, lane);
  pb.init(B, ldbu, n0, N, Ku, wave, lane);

  f32x4_t acc[TMI][TNJ];
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const bf16* As, const bf16* Bs) {
    i32x8_t a[TMI], b[TNJ];
#pragma unroll
    for (int j = 0; j < TNJ; ++j) b[j] = frag_f8<BN>(Bs, wn + 16 * j, lane);
#pragma unroll
    for (int i = 0; i < TMI; ++i) a[i] = frag_f8<BM>(As, wm + 16 * i, lane);
#pragma unroll
    for (int i = 0; i < TMI; ++i)
#pragma unroll
      for (int j = 0; j < TNJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], FB, FA,
                                                                     0, 0, 0, 0);
  };

  // per slice: wait until only A(s + 1) is in flight (loads land in issue
  // order), barrier (every wave is done with slice s - 1, whose stages the
  // next loads reuse), issue B(s + 1) then A(s + 2), multiply slice s
  const int nsl = (int)((kend - kbeg) / BK);
  bf16* const ra = lds;                    // A stages: ra + j BM 64
  bf16* const rb = lds + 3 * BM * 64;      // B stages: rb + j BN 64
  constexpr int NA = DmaPlan<BM, false>::NB;
  pa.issue(kbeg, ra, wave);
  pb.issue(kbeg, rb, wave);
  if (nsl > 1) pa.issue(kbeg + BK, ra + BM * 64, wave);
  int sa = 0, sb = 0;
  for (int it = 0; it < nsl; ++it) {
    if (it + 1 < nsl) dma_wait_n<NA>();
    else dma_wait();
    __syncthreads();
    const int sa2 = sa == 0 ? 2 : sa - 1;  // (it + 2) % 3
    if (it + 1 < nsl) pb.issue(kbeg + (int64_t)(it + 1) * BK, rb + (sb ^ 1) * BN * 64, wave);
    if (it + 2 < nsl) pa.issue(kbeg + (int64_t)(it + 2) * BK, ra + sa2 * BM * 64, wave);
    compute(ra + sa * BM * 64, rb + sb * BN * 64);
    sa = sa == 2 ? 0 : sa + 1;
    sb ^= 1;
  }
  const float sc = a_inv[0] * b_inv[0];
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNJ; ++j) acc[i][j] *= sc;
  store_tiles<EPI>(acc, M, N, m0 + wm, n0 + wn, lane, C, ldc, nullptr,
                   partial ? partial + (int64_t)split * M * N : nullptr);
}

// out[m, n] (=/+=) sum_s partial[s, m, n], fixed order over s
__global__ void k_splitk_reduce(const float* __restrict__ partial, int splits, int64_t M,
                                int64_t N, float* out, int64_t ldc, int accumulate) {
  const int64_t i = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * 4;
  const int64_t MN = M * N;
  if (i >= MN) return;
  f32x4_t s = *(const f32x4_t*)(partial + i);
  for (int k = 1; k < splits; ++k) s += *(const f32x4_t*)(partial + (int64_t)k * MN + i);
  const int64_t m = i / N, n = i % N;
  f32x4_t* o = (f32x4_t*)(out + m * ldc + n);
  if (accumulate) s += *o;
  *o = s;
}

// ------------------------------------------------------------------ host
bool mfma_gemm_supported(const GemmDesc& g) {
  if (g.K % 8 || g.lda % 8 || g.ldb % 8 || g.ldc % 4 || g.N % 4) return false;
  const bool TA = g.op == OP_TN, TB = g.op != OP_NT;
  if (TA && g.M % 8) return false;
  if (TB && g.N % 8) return false;
  const uintptr_t al = (uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)g.C |
                       (uintptr_t)(g.aux ? g.aux : g.C);
  if (al & 15) return false;
  return true;
}

// Algorithmic work of one product: 2 M N K flops; A and B read once, C
// written once (read too for RESADD / F32_ACC), aux read (DRELU2) once.  Split-K partials are the reduce kernel's traffic.
static Work gemm_work(const GemmDesc& g) {
  const double mn = (double)g.M * g.N;
  const bool f32out = g.epi == E_F32 || g.epi == E_F32_ACC;
  double bytes = 2.0 * ((double)g.M * g.K + (double)g.N * g.K) + mn * (f32out ? 4 : 2);
  if (g.epi == E_RESADD || g.epi == E_DRELU2) bytes += 2.0 * mn;
  if (g.epi == E_F32_ACC) bytes += 4.0 * mn;
  return Work(2.0 * mn * g.K, bytes);
}

template <int BM, int BN, bool TA, bool TB, int EPI>
static void launch(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int grid = ((nb + 7) / 8) * 8;
  GK_LAUNCH(gemm_work(g), (k_gemm_mfma<BM, BN, TA, TB, EPI>), dim3(grid), dim3(256), 0, s, g.M, g.N,
                     g.K, (const bf16*)g.A, g.lda, (const bf16*)g.B, g.ldb, g.C, g.ldc, g.aux, tm,
                     partial);
}

template <int BM, int BN, bool TA, bool TB>
static void launch_epi(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  switch (g.epi) {
    case E_STORE:   launch<BM, BN, TA, TB, E_STORE>(g, tm, partial, s); break;
    case E_RESADD:  launch<BM, BN, TA, TB, E_RESADD>(g, tm, partial, s); break;
    case E_RELU2:   launch<BM, BN, TA, TB, E_RELU2>(g, tm, partial, s); break;
    case E_DRELU2:  launch<BM, BN, TA, TB, E_DRELU2>(g, tm, partial, s); break;
    case E_F32:     launch<BM, BN, TA, TB, E_F32>(g, tm, partial, s); break;
    default:        launch<BM, BN, TA, TB, E_F32_ACC>(g, tm, partial, s); break;
  }
}

template <int BM, int BN>
static void launch_op(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  if (g.op == OP_NT) launch_epi<BM, BN, false, false>(g, tm, partial, s);
  else if (g.op == OP_NN) launch_epi<BM, BN, false, true>(g, tm, partial, s);
  else launch_epi<BM, BN, true, true>(g, tm, partial, s);
}

// Tile shape and K split of one product.  `scratch_bytes` bounds the split
// (SIZE_MAX: as the shape asks).
static TileMap plan(int64_t M, int64_t N, int64_t K, bool f32out, size_t scratch_bytes, int* bm) {
  const int kCU = 256;
  // 256x256 (one block per CU) when that still gives two full waves of
  // blocks; else 256x128 (two blocks per CU) unless that under-fills the chip
  int BM = 256, BN = 128;
  int64_t tiles = cdiv(M, 256) * cdiv(N, 128);
  if (cdiv(M, 256) * cdiv(N, 256) >= 2 * kCU) {
    BM = 512;            // code for the 256x256 kernel
    BN = 256;
    tiles = cdiv(M, 256) * cdiv(N, 256);
  } else if (tiles < 2 * kCU) {
    BM = 128; BN = 128; tiles = cdiv(M, 128) * cdiv(N, 128);
  }
  TileMap tm;
  tm.tiles_m = (int)cdiv(M, BM == 512 ? 256 : BM);
  tm.tiles_n = (int)cdiv(N, BN);
  tm.splits = 1;
  tm.k_per_split = cdiv(K, BK) * BK;
  if (f32out && tiles < kCU) {
    // split the reduction so the grid reaches ~2 blocks per CU, keeping at
    // least 8 K-slices per split
    const int64_t ksl = cdiv(K, BK);
    int sp = (int)cdiv(2 * kCU, tiles);
    sp = (int)std::min<int64_t>(sp, ksl / 8);
    sp = std::min(sp, 64);
    while (sp > 1 && (size_t)sp * M * N * 4 > scratch_bytes) --sp;
    if (sp > 1) {
      tm.k_per_split = cdiv(ksl, sp) * BK;
      tm.splits = (int)cdiv(K, tm.k_per_split);
    }
  }
  *bm = BM;
  return tm;
}

template <bool TA, bool TB, int EPI>
static void launch_db_t(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int grid = ((nb + 7) / 8) * 8;
  GK_LAUNCH(gemm_work(g), (k_gemm_mfma_db<TA, TB, EPI>), dim3(grid), dim3(512), 0, s, g.M, g.N, g.K,
                     (const bf16*)g.A, g.lda, (const bf16*)g.B, g.ldb, g.C, g.ldc, g.aux, tm,
                     partial);
}

template <bool TA, bool TB>
static void launch_db_e(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  switch (g.epi) {
    case E_STORE:   launch_db_t<TA, TB, E_STORE>(g, tm, partial, s); break;
    case E_RESADD:  launch_db_t<TA, TB, E_RESADD>(g, tm, partial, s); break;
    case E_RELU2:   launch_db_t<TA, TB, E_RELU2>(g, tm, partial, s); break;
    case E_DRELU2:  launch_db_t<TA, TB, E_DRELU2>(g, tm, partial, s); break;
    case E_F32:     launch_db_t<TA, TB, E_F32>(g, tm, partial, s); break;
    default:        launch_db_t<TA, TB, E_F32_ACC>(g, tm, partial, s); break;
  }
}

static void launch_db(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  if (g.op == OP_NT) launch_db_e<false, false>(g, tm, partial, s);
  else if (g.op == OP_NN) launch_db_e<false, true>(g, tm, partial, s);
  else launch_db_e<true, true>(g, tm, partial, s);
}

template <int BM, int BN, bool TA, bool TB, int EPI>
static void launch_dma_t(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int grid = ((nb + 7) / 8) * 8;
  GK_LAUNCH(gemm_work(g), (k_gemm_dma<BM, BN, TA, TB, EPI>), dim3(grid), dim3(512), 0, s, g.M,
            g.N, g.K, (const bf16*)g.A, g.lda, (const bf16*)g.B, g.ldb, g.C, g.ldc, g.aux, tm,
            partial);
}

template <int BM, int BN, bool TA, bool TB>
static void launch_dma_e(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  switch (g.epi) {
    case E_STORE:   launch_dma_t<BM, BN, TA, TB, E_STORE>(g, tm, partial, s); break;
    case E_RESADD:  launch_dma_t<BM, BN, TA, TB, E_RESADD>(g, tm, partial, s); break;
    case E_RELU2:   launch_dma_t<BM, BN, TA, TB, E_RELU2>(g, tm, partial, s); break;
    case E_DRELU2:  launch_dma_t<BM, BN, TA, TB, E_DRELU2>(g, tm, partial, s); break;
    case E_F32:     launch_dma_t<BM, BN, TA, TB, E_F32>(g, tm, partial, s); break;
    default:        launch_dma_t<BM, BN, TA, TB, E_F32_ACC>(g, tm, partial, s); break;
  }
}

template <int BM, int BN>
static void launch_dma(const GemmDesc& g, const TileMap& tm, float* partial, hipStream_t s) {
  if (g.op == OP_NT) launch_dma_e<BM, BN, false, false>(g, tm, partial, s);
  else if (g.op == OP_NN) launch_dma_e<BM, BN, false, true>(g, tm, partial, s);
  else launch_dma_e<BM, BN, true, true>(g, tm, partial, s);
}

// The direct-to-LDS kernel takes every product it can: K a multiple of 64,
// at least 2^31 multiply-adds (smaller ones keep the 4-wave kernels), and
// operands addressable with 32-bit buffer offsets.
static bool dma_shape_ok(int64_t M, int64_t N, int64_t K) {
  return K % BK == 0 && (double)M * N * K >= 2147483648.0;
}

static bool dma_ok(const GemmDesc& g) {
  if (!dma_shape_ok(g.M, g.N, g.K)) return false;
  const bool TA = g.op == OP_TN, TB = g.op != OP_NT;
  const double a_bytes = 2.0 * (TA ? g.K * g.lda : g.M * g.lda);
  const double b_bytes = 2.0 * (TB ? g.K * g.ldb : g.N * g.ldb);
  return a_bytes < 4294967295.0 && b_bytes < 4294967295.0;
}

// 256x256 tiles, one block per CU.  fp32 outputs may split K: the split
// minimises a time estimate, rounds of 256 blocks x K-slices per block x
// ~2.1 us per 256x256x64 slice, plus the partial tiles' HBM traffic (written
// and read once, ~5 TB/s) and the reduce launch; at least 8 K-slices per
// split.
static TileMap plan_dma(int64_t M, int64_t N, int64_t K, bool f32out, size_t scratch_bytes,
                        int* bn) {
  const int kCU = 256;
  TileMap tm;
  tm.tiles_m = (int)cdiv(M, 256);
  tm.tiles_n = (int)cdiv(N, 256);
  tm.splits = 1;
  tm.k_per_split = K;
  *bn = 256;
  if (!f32out) {
    // 256 x 192 tiles when they fill the rounds of 256 blocks better (N a
    // multiple of 192, e.g. 768 or 2304): fewer idle CUs in the last round
    if (N % 192 == 0) {
      const int64_t r256 = cdiv((int64_t)tm.tiles_m * tm.tiles_n, kCU) * 256;
      const int64_t r192 = cdiv((int64_t)tm.tiles_m * (N / 192), kCU) * 192;
      if (r192 < r256) {
        tm.tiles_n = (int)(N / 192);
        *bn = 192;
      }
    }
    return tm;
  }
  const int64_t tiles = (int64_t)tm.tiles_m * tm.tiles_n, ksl = K / BK;
  auto cost = [&](int sp) {
    const double rounds = (double)cdiv(tiles * sp, kCU);
    const double slices = (double)cdiv(ksl, sp);
    return rounds * slices * 2.1 + (sp > 1 ? sp * (double)M * N * 8.0 / 5e6 + 10.0 : 0.0);
  };
  int best = 1;
  double best_cost = cost(1);
  for (int sp = 2; sp <= 64 && ksl / sp >= 8; ++sp) {
    if ((size_t)sp * M * N * 4 > scratch_bytes) break;
    const double c = cost(sp);
    if (c < best_cost) { best = sp; best_cost = c; }
  }
  if (best > 1) {
    tm.k_per_split = cdiv(ksl, best) * BK;
    tm.splits = (int)cdiv(K, tm.k_per_split);
    // a split's run of tiles crosses XCDs: keep the larger operand's
    // panels (A's rows ~ M, B's ~ N) on one side of the cut
    tm.order = M >= N ? 1 : 2;
  }
  return tm;
}

bool qkv_rope_fused_ok(int64_t rows, int D, int H, int Hkv, int hd) {
  const int64_t n = (int64_t)(H + 2 * Hkv) * hd;
  return hd == 128 && rows >= 1 && D % BK == 0 && dma_shape_ok(rows, n, D) &&
         2.0 * rows * D < 4294967295.0 && 2.0 * n * D < 4294967295.0;
}

hipError_t qkv_gemm_rope_norm(const void* h, int64_t rows, int D, const void* wqkv, int H,
                              int Hkv, void* qkv, const float* cs, float* rq, float* rk, int T,
                              float eps, const VeArgs* ve, hipStream_t s) {
  if (!qkv_rope_fused_ok(rows, D, H, Hkv, 128)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)(H + 2 * Hkv) * 128;
  TileMap tm;
  tm.tiles_m = (int)cdiv(rows, 256);
  tm.tiles_n = (int)cdiv(n, 256);
  tm.splits = 1;
  tm.k_per_split = D;
  tm.qk_cs = (const float2*)cs;
  tm.qk_rq = rq;
  tm.qk_rk = rk;
  tm.qk_T = T;
  tm.qk_H = H;
  tm.qk_Hkv = Hkv;
  tm.qk_eps = eps;
  if (ve) {
    tm.ve_tok = ve->tok;
    tm.ve_h = (const bf16*)h;
    tm.ve_D = D;
    tm.ve_wg = (const bf16*)ve->wg;
    tm.ve_C = ve->C;
    tm.ve_E = (const bf16*)ve->E;
    tm.ve_g = ve->g;
  }
  const int nb = tm.tiles_m * tm.tiles_n;
  const int grid = ((nb + 7) / 8) * 8;
  // 2 rows n D flops; h and Wqkv read once, qkv written once, 1/rms written
  const Work w(2.0 * rows * n * D, 2.0 * ((double)rows * D + (double)n * D + (double)rows * n) +
                                       4.0 * rows * (H + Hkv));
  GK_LAUNCH(w, (k_gemm_dma<256, 256, false, false, E_QKNORM>), dim3(grid), dim3(512), 0, s, rows,
            n, (int64_t)D, (const bf16*)h, (int64_t)D, (const bf16*)wqkv, (int64_t)D, qkv, n,
            nullptr, tm, nullptr);
  return hipGetLastError();
}

// any row count (partial row tiles read zeros past the last row)
bool lm_ce_fused_ok(int64_t rows, int V, int D) {
  return rows >= 1 && V % 256 == 0 && V / 256 <= 1024 && D % BK == 0 &&
         2.0 * rows * D < 4294967295.0 && 2.0 * V * D < 4294967295.0;
}

// e [rows, V] addressable with 32-bit buffer offsets
bool lm_ce_bwd_ok(int64_t rows, int V, int D) {
  return lm_ce_fused_ok(rows, V, D) && 2.0 * rows * V < 4294967295.0;
}

size_t lm_ce_stats_bytes(int64_t rows, int V) { return (size_t)rows * (V / 256) * 8; }

hipError_t lm_ce_gemm(const void* hf, int64_t rows, int D, const void* wlm, int V, void* e,
                      float* stats, float* zt, const int32_t* tok, int tgt_T, int tgt_direct,
                      hipStream_t s) {
  if (!lm_ce_fused_ok(rows, V, D)) return hipErrorInvalidValue;
  TileMap tm;
  tm.tiles_m = (int)cdiv(rows, 256);
  tm.tiles_n = V / 256;
  tm.splits = 1;
  tm.k_per_split = D;
  tm.ce_stats = stats;
  tm.ce_zt = zt;
  tm.ce_tok = tok;
  tm.ce_T = tgt_T;
  tm.ce_direct = tgt_direct;
  const int nb = tm.tiles_m * tm.tiles_n;
  const int grid = ((nb + 7) / 8) * 8;
  // 2 rows V D flops; hf and Wlm read once, e written (2 bytes), stats and
  // target logits written
  const double mn = (double)rows * V;
  const Work w(2.0 * mn * D, 2.0 * ((double)rows * D + (double)V * D) + (e ? 2.0 * mn : 0.0) +
                                 8.0 * rows * (V / 256) + 4.0 * rows);
  GK_LAUNCH(w, (k_gemm_dma<256, 256, false, false, E_CE>), dim3(grid), dim3(512), 0, s, rows,
            (int64_t)V, (int64_t)D, (const bf16*)hf, (int64_t)D, (const bf16*)wlm, (int64_t)D,
            e, (int64_t)V, nullptr, tm, nullptr);
  return hipGetLastError();
}

hipError_t lm_ce_bwd_gemm(const void* e, int64_t rows, int V, const void* wlm, int D, void* dh,
                          const float* stats, const float* lse, const int32_t* tok, int tgt_T,
                          int tgt_direct, float grad_scale, hipStream_t s) {
  if (!lm_ce_bwd_ok(rows, V, D)) return hipErrorInvalidValue;
  // 256 x 192 tiles whatever D is (the 256-wide tile's extra per-row state
  // would not fit its registers); columns past D are dropped
  TileMap tm;
  tm.tiles_m = (int)cdiv(rows, 256);
  tm.tiles_n = (int)cdiv(D, 192);
  tm.splits = 1;
  tm.k_per_split = V;
  tm.ce_stats = (float*)stats;
  tm.ce_tok = tok;
  tm.ce_T = tgt_T;
  tm.ce_direct = tgt_direct;
  tm.ce_lse = lse;
  tm.ce_scale = grad_scale;
  const int nb = tm.tiles_m * tm.tiles_n;
  const int grid = ((nb + 7) / 8) * 8;
  // 2 rows D V flops; e and Wlm read once, dh written, the stats' maxima,
  // lse, the targets and their Wlm rows read
  const Work w(2.0 * rows * D * V, 2.0 * ((double)rows * V + (double)V * D + 2.0 * rows * D) +
                                       4.0 * rows * (V / 256 + 2));
  GK_LAUNCH(w, (k_gemm_dma<256, 192, false, true, E_CEB>), dim3(grid), dim3(512), 0, s, rows,
            (int64_t)D, (int64_t)V, (const bf16*)e, (int64_t)V, (const bf16*)wlm, (int64_t)D, dh,
            (int64_t)D, nullptr, tm, nullptr);
  return hipGetLastError();
}

size_t mfma_splitk_bytes(int64_t M, int64_t N, int64_t K) {
  int bm;
  TileMap tm = plan(M, N, K, true, SIZE_MAX, &bm);
  size_t b = tm.splits > 1 ? (size_t)tm.splits * M * N * sizeof(float) : 0;
  if (dma_shape_ok(M, N, K)) {
    int bn;
    TileMap td = plan_dma(M, N, K, true, SIZE_MAX, &bn);
    if (td.splits > 1) b = std::max(b, (size_t)td.splits * M * N * sizeof(float));
  }
  return b;
}

hipError_t mfma_gemm(const GemmDesc& g, hipStream_t s) {
  const bool f32out = g.epi == E_F32 || g.epi == E_F32_ACC;
  const size_t scr = g.scratch ? g.scratch_bytes : 0;
  TileMap tm;
  float* partial = nullptr;
  if (dma_ok(g)) {
    int bn;
    tm = plan_dma(g.M, g.N, g.K, f32out, scr, &bn);
    partial = tm.splits > 1 ? (float*)g.scratch : nullptr;
    if (bn == 192) launch_dma<256, 192>(g, tm, partial, s);
    else launch_dma<256, 256>(g, tm, partial, s);
  } else {
    int BM;
    tm = plan(g.M, g.N, g.K, f32out, scr, &BM);
    partial = tm.splits > 1 ? (float*)g.scratch : nullptr;
    if (BM == 512) launch_db(g, tm, partial, s);
    else if (BM == 256) launch_op<256, 128>(g, tm, partial, s);
    else launch_op<128, 128>(g, tm, partial, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !partial) return e;
  const int64_t MN = g.M * g.N;
  const Work rw(0.0, 4.0 * MN * (tm.splits + 1 + (g.epi == E_F32_ACC ? 1 : 0)));
  GK_LAUNCH(rw, k_splitk_reduce, dim3((unsigned)cdiv(MN / 4, 256)), dim3(256), 0, s, partial,
            tm.splits, g.M, g.N, (float*)g.C, g.ldc, g.epi == E_F32_ACC ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gk

namespace gk {

template <int BN, int FA, int FB, int EPI>
static void launch_fp8_t(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         const void* B, int64_t ldb, const float* ai, const float* bi, void* C,
                         int64_t ldc, const TileMap& tm, float* partial, hipStream_t s) {
  const int nb = tm.tiles_m * tm.tiles_n * tm.splits;
  const int grid = ((nb + 7) / 8) * 8;
  const double mn = (double)M * N;
  const Work w(2.0 * mn * K, (double)M * K + (double)N * K +
                                 mn * (EPI == E_STORE ? 2 : EPI == E_F32 ? 4 : 8));
  GK_LAUNCH(w, (k_gemm_fp8<BN, FA, FB, EPI>), dim3(grid), dim3(512), 0, s, M, N, K / 2,
            (const bf16*)A, lda / 2, (const bf16*)B, ldb / 2, ai, bi, C, ldc, tm, partial);
}

template <int BN, int FA, int FB>
static void launch_fp8_e(int epi, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         const void* B, int64_t ldb, const float* ai, const float* bi, void* C,
                         int64_t ldc, const TileMap& tm, float* partial, hipStream_t s) {
  if (partial || epi == E_F32)
    launch_fp8_t<BN, FA, FB, E_F32>(M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
  else if (epi == E_F32_ACC)
    launch_fp8_t<BN, FA, FB, E_F32_ACC>(M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
  else
    launch_fp8_t<BN, FA, FB, E_STORE>(M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
}

template <int BN>
static void launch_fp8_f(int fa, int fb, int epi, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, const void* B, int64_t ldb, const float* ai,
                         const float* bi, void* C, int64_t ldc, const TileMap& tm, float* partial,
                         hipStream_t s) {
  if (fa == 0 && fb == 0)
    launch_fp8_e<BN, 0, 0>(epi, M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
  else if (fa == 1 && fb == 0)
    launch_fp8_e<BN, 1, 0>(epi, M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
  else if (fa == 0 && fb == 1)
    launch_fp8_e<BN, 0, 1>(epi, M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
  else
    launch_fp8_e<BN, 1, 1>(epi, M, N, K, A, lda, B, ldb, ai, bi, C, ldc, tm, partial, s);
}

bool gemm_fp8_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
  return M >= 1 && N >= 1 && K >= 128 && K % 128 == 0 && lda >= K && ldb >= K && lda % 16 == 0 &&
         ldb % 16 == 0 && ldc >= N && ldc % 4 == 0 && N % 4 == 0 &&
         (double)M * lda < 4294967295.0 && (double)N * ldb < 4294967295.0;
}

size_t gemm_fp8_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  int bn;
  const TileMap tm = plan_dma(M, N, K / 2, true, SIZE_MAX, &bn);
  return tm.splits > 1 ? (size_t)tm.splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                    const void* B, int64_t ldb, int fb, const float* a_inv, const float* b_inv,
                    void* C, int64_t ldc, int epi, void* scratch, size_t scratch_bytes,
                    hipStream_t s) {
  if (!gemm_fp8_ok(M, N, K, lda, ldb, ldc)) return hipErrorInvalidValue;
  const bool f32out = epi == E_F32 || epi == E_F32_ACC;
  int bn;
  const TileMap tm = plan_dma(M, N, K / 2, f32out, scratch ? scratch_bytes : 0, &bn);
  float* partial = tm.splits > 1 ? (float*)scratch : nullptr;
  if (bn == 192)
    launch_fp8_f<192>(fa, fb, epi, M, N, K, A, lda, B, ldb, a_inv, b_inv, C, ldc, tm, partial, s);
  else
    launch_fp8_f<256>(fa, fb, epi, M, N, K, A, lda, B, ldb, a_inv, b_inv, C, ldc, tm, partial, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !partial) return e;
  const int64_t MN = M * N;
  const Work rw(0.0, 4.0 * MN * (tm.splits + 1 + (epi == E_F32_ACC ? 1 : 0)));
  GK_LAUNCH(rw, k_splitk_reduce, dim3((unsigned)cdiv(MN / 4, 256)), dim3(256), 0, s, partial,
            tm.splits, M, N, (float*)C, ldc, epi == E_F32_ACC ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gk

namespace gk {

template <int BM, int BN, bool TA, bool TB, int EPI>
static void launch_batched_t(const GemmDesc& g, TileMap tm, int batch, hipStream_t s) {
  tm.batch = batch;
  const int64_t nb = (int64_t)tm.tiles_m * tm.tiles_n * batch;
  const int grid = (int)(((nb + 7) / 8) * 8);
  Work w = gemm_work(g);
  w.flops *= batch;
  w.bytes *= batch;
  GK_LAUNCH(w, (k_gemm_mfma<BM, BN, TA, TB, EPI>), dim3(grid), dim3(256), 0, s, g.M, g.N, g.K,
            (const bf16*)g.A, g.lda, (const bf16*)g.B, g.ldb, g.C, g.ldc, nullptr, tm, nullptr);
}

template <int BM, int BN, int EPI>
static void launch_batched_op(const GemmDesc& g, const TileMap& tm, int batch, hipStream_t s) {
  if (g.op == OP_NT) launch_batched_t<BM, BN, false, false, EPI>(g, tm, batch, s);
  else if (g.op == OP_NN) launch_batched_t<BM, BN, false, true, EPI>(g, tm, batch, s);
  else launch_batched_t<BM, BN, true, true, EPI>(g, tm, batch, s);
}

// `batch` products of one shape with A, B, C advanced by sa, sb, sc elements
// per product (bf16 operands, E_STORE or E_F32, no K split): the direct-to-
// LDS kernel when the product suits it (K a multiple of 64, at least 2^32
// multiply-adds and a round of 256 x 256 tiles over the batch), else the
// 4-wave kernel, 256 x 128 tiles
// when the batch gives two rounds of them, else 128 x 128.
hipError_t gemm_batched(const GemmDesc& g, int batch, int64_t sa, int64_t sb, int64_t sc,
                        hipStream_t s) {
  if (batch < 1 || batch > 65535 || !mfma_gemm_supported(g) ||
      (g.epi != E_STORE && g.epi != E_F32))
    return hipErrorInvalidValue;
  const bool TA = g.op == OP_TN, TB = g.op != OP_NT;
  const double a_bytes = 2.0 * (TA ? g.K * g.lda : g.M * g.lda);
  const double b_bytes = 2.0 * (TB ? g.K * g.ldb : g.N * g.ldb);
  if (g.K % BK == 0 && a_bytes < 4294967295.0 && b_bytes < 4294967295.0 &&
      (double)g.M * g.N * g.K * batch >= 4294967296.0 &&
      cdiv(g.M, 256) * cdiv(g.N, 256) * batch >= 256) {
    // the direct-to-LDS kernel, 256 x 256 tiles
    TileMap tm;
    tm.tiles_m = (int)cdiv(g.M, 256);
    tm.tiles_n = (int)cdiv(g.N, 256);
    tm.splits = 1;
    tm.k_per_split = g.K;
    tm.bs_a = sa;
    tm.bs_b = sb;
    tm.bs_c = sc;
    tm.batch = batch;
    const int64_t nb = (int64_t)tm.tiles_m * tm.tiles_n * batch;
    const dim3 grid((unsigned)(((nb + 7) / 8) * 8));
    Work w = gemm_work(g);
    w.flops *= batch;
    w.bytes *= batch;
#define GK_DMA_B(TA, TB, EPI)                                                                   \
  GK_LAUNCH(w, (k_gemm_dma<256, 256, TA, TB, EPI>), grid, dim3(512), 0, s, g.M, g.N, g.K,       \
            (const bf16*)g.A, g.lda, (const bf16*)g.B, g.ldb, g.C, g.ldc, nullptr, tm, nullptr)
    if (g.epi == E_STORE) {
      if (g.op == OP_NT) GK_DMA_B(false, false, E_STORE);
      else if (g.op == OP_NN) GK_DMA_B(false, true, E_STORE);
      else GK_DMA_B(true, true, E_STORE);
    } else {
      if (g.op == OP_NT) GK_DMA_B(false, false, E_F32);
      else if (g.op == OP_NN) GK_DMA_B(false, true, E_F32);
      else GK_DMA_B(true, true, E_F32);
    }
#undef GK_DMA_B
    return hipGetLastError();
  }
  const bool big = cdiv(g.M, 256) * cdiv(g.N, 128) * batch >= 2 * 256;
  TileMap tm;
  tm.tiles_m = (int)cdiv(g.M, big ? 256 : 128);
  tm.tiles_n = (int)cdiv(g.N, 128);
  tm.splits = 1;
  tm.k_per_split = cdiv(g.K, BK) * BK;
  tm.bs_a = sa;
  tm.bs_b = sb;
  tm.bs_c = sc;
  if (big) {
    if (g.epi == E_STORE) launch_batched_op<256, 128, E_STORE>(g, tm, batch, s);
    else launch_batched_op<256, 128, E_F32>(g, tm, batch, s);
  } else {
    if (g.epi == E_STORE) launch_batched_op<128, 128, E_STORE>(g, tm, batch, s);
    else launch_batched_op<128, 128, E_F32>(g, tm, batch, s);
  }
  return hipGetLastError();
}

}  // namespace gk
