// Shared tile plumbing of the head_dim-128 MFMA attention kernels (gfx950).
//
// Conventions
//   MFMA: v_mfma_f32_16x16x32_bf16, D[i][j] = sum_k X[i][k] Y[k][j].  Lane l
//   (g = l / 16, c = l % 16) supplies X row c and Y column c, 8 k-values each
//   (the same 8 k-slots for X and Y), and receives D[4g + r][c], r = 0..3.
//
//   Row-major tiles ("R" tiles, [rows][128 + 8] bf16) feed MFMA operands
//   whose contraction index is head_dim.
//
//   Transposed tiles ("T" tiles, [128][64 + 8] bf16) hold a [64 rows][128]
//   block as [hd][row], with the 64 rows permuted inside each 32-row chunk:
//   row 16*blk + 4*g + r (blk, r < 2, 4) sits at position 8*g + 4*blk + r.
//   A lane of group g then reads its 8 contraction values as one 16-byte run
//   at position 8*g, and those are exactly the rows 4g..4g+3 and 16+4g..16+4g+3
//   whose values an MFMA accumulator pair hands that lane (D rows 4g + r of
//   two 16-row blocks).  Probabilities or score gradients therefore go from
//   accumulators to the next MFMA without an LDS round trip.
#pragma once
#include "common.h"

namespace gk {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int HD = 128;
constexpr int TR = 64;            // rows per staged tile
constexpr int LDR = HD + 8;       // R-tile row stride (elements)
constexpr int LDT = TR + 8;       // T-tile row stride (elements)

__device__ __forceinline__ f32x4_t mfma(bf16x8_t x, bf16x8_t y, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Pack two accumulator quads (8 fp32) into one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8_t pack8(f32x4_t a, f32x4_t b) {
  uint4 u;
  u.x = pack2bf(a[0], a[1]);
  u.y = pack2bf(a[2], a[3]);
  u.z = pack2bf(b[0], b[1]);
  u.w = pack2bf(b[2], b[3]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// Global rows [row0, row0 + 64) of a [T][ld] matrix (128 columns from col0),
// fetched by NT threads into registers; rows >= T read as zero.
template <int NT>
struct TileRegs {
  static constexpr int NV = TR * HD / 8 / NT;      // uint4 per thread
  uint4 v[NV];
  __device__ __forceinline__ void load_rows(const bf16* g, int64_t ld, int row0, int T) {
    // chunk c: row c / 16, 8-column group c % 16
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c >> 4, ch = c & 15;
      v[i] = row0 + r < T ? *(const uint4*)(g + (int64_t)(row0 + r) * ld + ch * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_rows(bf16* s) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c >> 4, ch = c & 15;
      *(uint4*)(s + r * LDR + ch * 8) = v[i];
    }
  }
  // patch p (8 rows x 8 columns): rows 8*(p / 16).., columns 8*(p % 16)..
  __device__ __forceinline__ void load_patches(const bf16* g, int64_t ld, int row0, int T) {
    constexpr int NP = TR * HD / 64 / NT;            // patches per thread
    static_assert(NV == 8 * NP, "patch count");
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
      const int p = threadIdx.x + NT * pi;
      const int rb = p >> 4, cb = p & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = row0 + rb * 8 + e;
        v[pi * 8 + e] = row < T ? *(const uint4*)(g + (int64_t)row * ld + cb * 8)
                                : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store_patches_T(bf16* s) const {
    constexpr int NP = TR * HD / 64 / NT;
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
      const int p = threadIdx.x + NT * pi;
      const int rb = p >> 4, cb = p & 15;
      // rows 8*rb + e of the tile: chunk rb/4, 8-row group q = rb%4 inside it
      const int q = rb & 3;
      const int base0 = 32 * (rb >> 2) + 16 * (q & 1) + 4 * (q >> 1);
      const uint32_t* w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (const uint32_t*)&v[pi * 8 + e];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint2 lo0, hi0, lo1, hi1;
        lo0.x = lo_pair(w[0][d], w[1][d]); hi0.x = hi_pair(w[0][d], w[1][d]);
        lo0.y = lo_pair(w[2][d], w[3][d]); hi0.y = hi_pair(w[2][d], w[3][d]);
        lo1.x = lo_pair(w[4][d], w[5][d]); hi1.x = hi_pair(w[4][d], w[5][d]);
        lo1.y = lo_pair(w[6][d], w[7][d]); hi1.y = hi_pair(w[6][d], w[7][d]);
        bf16* c0 = s + (cb * 8 + 2 * d) * LDT;
        bf16* c1 = c0 + LDT;
        *(uint2*)(c0 + base0) = lo0;
        *(uint2*)(c0 + base0 + 8) = lo1;
        *(uint2*)(c1 + base0) = hi0;
        *(uint2*)(c1 + base0 + 8) = hi1;
      }
    }
  }
};

// 8 contraction values of an R tile: row `row`, head-dim slots 32*ks + 8g.
__device__ __forceinline__ bf16x8_t rfrag(const bf16* s, int row, int ks, int g) {
  return *(const bf16x8_t*)(s + row * LDR + 32 * ks + 8 * g);
}
// 8 contraction values of a T tile: head-dim row `hrow`, 32-row chunk `ch`.
__device__ __forceinline__ bf16x8_t tfrag(const bf16* s, int hrow, int ch, int g) {
  return *(const bf16x8_t*)(s + hrow * LDT + 32 * ch + 8 * g);
}

}  // namespace attn
}  // namespace gk
