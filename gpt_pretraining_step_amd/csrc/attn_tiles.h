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
#include "dma.h"

namespace gk {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int HD = 128;
constexpr int TR = 64;            // rows per staged tile
constexpr int LDR = HD + 8;       // R-tile row stride (elements)
constexpr int LDT = TR + 8;       // T-tile row stride (elements)

// T-tile element offset of (head-dim row, position): 8-element chunks XOR-
// swizzled by (row / 16) % 8 so the transposing writes (lanes 8 rows apart)
// spread over the banks; reads of 16 consecutive rows stay conflict-free.
__device__ __forceinline__ int toff(int row, int pos) {
  return row * LDT + ((((pos >> 3) ^ (row >> 4)) & 7) << 3) + (pos & 7);
}

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

// Global rows [row0, row0 + 64) of a [T][ld] matrix (128 columns), fetched
// by NT threads into registers; rows >= T read as zero.  Either as 16-byte
// row chunks (store_rows) or as PR x 8 patches (PR = 8 for 128 threads, 4
// for 256), which can be written both as an R tile and, transposed, as a T
// tile.
template <int NT>
struct TileRegs {
  static constexpr int NV = TR * HD / 8 / NT;      // uint4 per thread
  static constexpr int PR = NV;                    // patch rows: one patch per thread
  static_assert(PR == 8 || PR == 4, "128 or 256 threads");
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
  // patch of this thread: rows PR*(tid / 16) + e, columns 8*(tid % 16)..
  __device__ __forceinline__ void load_patches(const bf16* g, int64_t ld, int row0, int T) {
    const int rb = threadIdx.x >> 4, cb = threadIdx.x & 15;
#pragma unroll
    for (int e = 0; e < PR; ++e) {
      const int row = row0 + rb * PR + e;
      v[e] = row < T ? *(const uint4*)(g + (int64_t)row * ld + cb * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_patches_R(bf16* s) const {
    const int rb = threadIdx.x >> 4, cb = threadIdx.x & 15;
#pragma unroll
    for (int e = 0; e < PR; ++e) *(uint4*)(s + (rb * PR + e) * LDR + cb * 8) = v[e];
  }
  __device__ __forceinline__ void store_patches_T(bf16* s) const {
    const int rb = threadIdx.x >> 4, cb = threadIdx.x & 15;
    const uint32_t* w[PR];
#pragma unroll
    for (int e = 0; e < PR; ++e) w[e] = (const uint32_t*)&v[e];
    // position of tile row j (inside its 32-row chunk): 8 g + 4 blk + r for
    // j = 16 blk + 4 g + r; the patch rows form runs of 4 consecutive positions
    int base0;
    if constexpr (PR == 8) {
      const int q = rb & 3;                         // 8-row group inside the chunk
      base0 = 32 * (rb >> 2) + 16 * (q & 1) + 4 * (q >> 1);
    } else {
      const int q = rb & 7;                         // 4-row group inside the chunk
      base0 = 32 * (rb >> 3) + 8 * (q & 3) + 4 * (q >> 2);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r0 = cb * 8 + 2 * d;
#pragma unroll
      for (int run = 0; run < PR / 4; ++run) {
        uint2 lo, hi;
        lo.x = lo_pair(w[4 * run][d], w[4 * run + 1][d]);
        hi.x = hi_pair(w[4 * run][d], w[4 * run + 1][d]);
        lo.y = lo_pair(w[4 * run + 2][d], w[4 * run + 3][d]);
        hi.y = hi_pair(w[4 * run + 2][d], w[4 * run + 3][d]);
        *(uint2*)(s + toff(r0, base0 + 8 * run)) = lo;
        *(uint2*)(s + toff(r0 + 1, base0 + 8 * run)) = hi;
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
  return *(const bf16x8_t*)(s + toff(hrow, 32 * ch + 8 * g));
}


// ------------------------------------------------ buffer-to-LDS staged tiles
// A [64 rows][128] tile as it sits in memory (256-byte rows, no padding),
// filled by buffer loads straight into LDS.  The 16-byte chunk c of row r
// is stored at chunk position c ^ dsw(r).  A 16-byte fragment read is served
// 32 lanes (512 bytes) at a time: 16 rows x 2 adjacent chunks, so the rows of
// each parity need distinct dsw(r) / 2; a transposing read covers 8
// consecutive rows x 32 bytes, which needs dsw(r) / 2 distinct over aligned
// groups of 8 rows.  dsw(r) = 2 ((r & 7) ^ ((r >> 3) & 1)) meets both (the
// hardware's bank-conflict counter reads 0 for both reads of this layout).
__device__ __forceinline__ int dsw(int r) { return 2 * ((r & 7) ^ ((r >> 3) & 1)); }
__device__ __forceinline__ int doff(int r, int col) {
  return r * HD + 8 * ((col >> 3) ^ dsw(r)) + (col & 7);
}

// Loads rows [row0, row0 + 64) of a [T][ld] bf16 matrix (128 columns from
// `base`) into a tile with the 4 waves of a workgroup: 4 x 1 KB per wave.
// Rows at or past T read as zeros.
struct TileDma {
  uint32_t voff, ldb;
  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
    ldb = (uint32_t)(ld * 2);
    const int row = 4 * wave + (lane >> 4), p = lane & 15;
    voff = (uint32_t)row * ldb + 16u * (uint32_t)(p ^ dsw(row));
  }
  __device__ __forceinline__ void issue(const bf16* base, int T, int row0, bf16* tile,
                                        int wave) const {
    const i32x4_t rsrc = make_rsrc(base, ((int64_t)(T - 1) * (ldb / 2) + HD) * 2);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)tile + 1024u * (uint32_t)wave);
    const uint32_t s0 = (uint32_t)row0 * ldb;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rsrc, lds + 4096u * i, voff + s0 + 16u * ldb * i);
  }
};

// 64 consecutive floats v[row0 ..] of a length-T vector into LDS (one wave,
// one 1 KB block: lanes 0..15 carry the data, the rest write zeros after
// it).  Entries at or past T read as zeros.
__device__ __forceinline__ void dma_vec64(const float* v, int T, int row0, float* dst, int lane) {
  const i32x4_t rsrc = make_rsrc(v, (int64_t)T * 4);
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)dst);
  const uint32_t off = lane < 16 ? (uint32_t)row0 * 4u + 16u * (uint32_t)lane : 0xFFFFFFF0u;
  dma16(rsrc, lds, off);
}

// 8 contraction values along the columns: row `row`, columns 32 ks + 8 g ..
__device__ __forceinline__ bf16x8_t dfrag_row(const bf16* t, int row, int ks, int g) {
  return *(const bf16x8_t*)(t + doff(row, 32 * ks + 8 * g));
}

// 8 contraction values along the rows for column c0 + (lane % 16): rows
// ka .. ka+3 then kb .. kb+3 (two transposing reads).
__device__ __forceinline__ bf16x8_t dfrag_col(const bf16* t, int c0, int ka, int kb, int l16) {
  const int r = l16 >> 2, c = c0 + 4 * (l16 & 3);
  const v4s_t x = tr16(t + doff(ka + r, c));
  const v4s_t y = tr16(t + doff(kb + r, c));
  typedef short v8s_t __attribute__((ext_vector_type(8)));
  const v8s_t v = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace attn
}  // namespace gk
