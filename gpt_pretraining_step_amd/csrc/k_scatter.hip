// Deterministic gradient scatter into the embedding tables (token embedding
// and value embeddings): dst[v, :] (=/+=) sum over the positions n holding
// token v of f(n, col) * src[n, col].
//
// The token ids of a batch are sorted once per backward pass (keys
// (id << 32) | n, so the order is unique): 1024-key runs are bitonic-sorted
// in LDS, then merged pairwise (each element finds its place in the partner
// run by binary search).  A segment table gives each id its range in the
// sorted order.  The sums are then taken over fixed 64-position chunks of the
// sorted order: a run of one id that lies inside a chunk and is the whole
// segment is written directly; runs cut by chunk boundaries leave partial
// rows that a second kernel adds in chunk order.  Every sum has a fixed order:
// the result does not depend on scheduling (no atomics), and a frequent id's
// thousands of rows are spread over many blocks.
#include <stdint.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {

static constexpr int kRun = 1024;     // keys per first-pass block
static constexpr int kChunk = 64;     // sorted positions per row-sum block
static constexpr uint64_t kPad = ~0ull;

#define TRY_K(x)                      \
  do {                                \
    const hipError_t e_ = (x);        \
    if (e_ != hipSuccess) return e_;  \
  } while (0)

struct SortLayout {
  int64_t npad;
  int rounds;                        // merge rounds; the sorted keys end in keys[rounds % 2]
  size_t keys[2], first, last, part, total;
};

static SortLayout sort_layout(int64_t N, int V, int maxW) {
  SortLayout L;
  L.npad = cdiv(N, kRun) * kRun;
  L.rounds = 0;
  for (int64_t run = kRun; run < L.npad; run <<= 1) ++L.rounds;
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o += (b + 255) / 256 * 256;
    return at;
  };
  L.keys[0] = take((size_t)L.npad * 8);
  L.keys[1] = take((size_t)L.npad * 8);
  L.first = take((size_t)V * 4);
  L.last = take((size_t)V * 4);
  L.part = take((size_t)cdiv(N, kChunk) * 2 * maxW * 4);
  L.total = o;
  return L;
}

size_t tok_sort_bytes(int64_t N, int V, int maxW) { return sort_layout(N, V, maxW).total; }

// ---- sort -------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sort_runs(const int32_t* tok, int T, int64_t N,
                                                   uint64_t* keys) {
  __shared__ uint64_t s[kRun];
  const int64_t base = (int64_t)blockIdx.x * kRun;
  for (int t = threadIdx.x; t < kRun; t += blockDim.x) {
    const int64_t n = base + t;
    s[t] = n < N ? ((uint64_t)(uint32_t)tok[(n / T) * (T + 1) + n % T] << 32) | (uint64_t)n
                 : kPad;
  }
  __syncthreads();
  for (int k = 2; k <= kRun; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = threadIdx.x; p < kRun / 2; p += blockDim.x) {
        const int i = 2 * p - (p & (j - 1));        // lower index of the pair (bit j clear)
        const int l = i + j;
        const bool up = (i & k) == 0;
        const uint64_t a = s[i], b = s[l];
        if ((a > b) == up) {
          s[i] = b;
          s[l] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int t = threadIdx.x; t < kRun; t += blockDim.x) keys[base + t] = s[t];
}

// Merge runs of length L pairwise: an element's place is its index in its run
// plus the number of partner-run keys below it (left run) or not above it
// (right run), which keeps equal keys (padding) stable.
__global__ __launch_bounds__(256) void k_merge_runs(const uint64_t* in, uint64_t* out,
                                                    int64_t npad, int64_t L) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= npad) return;
  const int64_t r = idx / L, pos = idx % L;
  const uint64_t key = in[idx];
  const int64_t pb = (r ^ 1) * L;
  int64_t cnt = 0;
  if (pb < npad) {
    int64_t lo = 0, hi = std::min(L, npad - pb);
    const bool left = (r & 1) == 0;
    while (lo < hi) {                                  // first partner key >= / > key
      const int64_t mid = (lo + hi) >> 1;
      const uint64_t v = in[pb + mid];
      if (left ? v < key : v <= key) lo = mid + 1;
      else hi = mid;
    }
    cnt = lo;
  }
  out[(r & ~(int64_t)1) * L + pos + cnt] = key;
}

// first1[id] / last1[id] = 1 + first / last sorted index of id (0: absent)
__global__ __launch_bounds__(256) void k_segments(const uint64_t* keys, int64_t N,
                                                  int32_t* first1, int32_t* last1) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= N) return;
  const uint32_t id = (uint32_t)(keys[i] >> 32);
  if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != id) first1[id] = (int32_t)(i + 1);
  if (i == N - 1 || (uint32_t)(keys[i + 1] >> 32) != id) last1[id] = (int32_t)(i + 1);
}

hipError_t tok_sort(const int32_t* tok, int B, int T, int V, int maxW, void* scratch,
                    hipStream_t s) {
  const int64_t N = (int64_t)B * T;
  const SortLayout L = sort_layout(N, V, maxW);
  char* base = (char*)scratch;
  uint64_t* k0 = (uint64_t*)(base + L.keys[0]);
  uint64_t* k1 = (uint64_t*)(base + L.keys[1]);
  GK_LAUNCH(Work(0.0, N * 12.0), k_sort_runs, dim3((unsigned)(L.npad / kRun)), dim3(256), 0, s,
            tok, T, N, k0);
  for (int64_t run = kRun; run < L.npad; run <<= 1) {
    GK_LAUNCH(Work(), k_merge_runs, dim3((unsigned)cdiv(L.npad, 256)), dim3(256), 0, s, k0, k1,
              L.npad, run);
    std::swap(k0, k1);
  }
  TRY_K(fill_zero(base + L.first, (int64_t)V * 4, s));
  TRY_K(fill_zero(base + L.last, (int64_t)V * 4, s));
  GK_LAUNCH(Work(), k_segments, dim3((unsigned)cdiv(N, 256)), dim3(256), 0, s,
            (const uint64_t*)(base + L.keys[L.rounds & 1]), N, (int32_t*)(base + L.first),
            (int32_t*)(base + L.last));
  return hipGetLastError();
}

// ---- row sums ---------------------------------------------------------------
// Columns in passes of 256: lane l of a wave holds 4 consecutive columns of
// each pass.
static constexpr int kMaxPass = 8;    // W <= 2048

template <typename Tv>
__device__ __forceinline__ void load4(const Tv* p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<bf16>(const bf16* p, float (&v)[4]) {
  const uint2 u = *(const uint2*)p;
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
  const float4 u = *(const float4*)p;
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}

// Sum of rows [i0, i1) of the chunk (sorted order) into acc, loads issued in
// groups of 4 rows.
template <typename Tv, int NP>
__device__ __forceinline__ void rows_sum(const uint64_t* ck, int i0, int i1, const Tv* src,
                                         int64_t ld, int W, const float* gate, int Hkv, int hd,
                                         int lane, float (&acc)[NP][4]) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[p][e] = 0.f;
  for (int b = i0; b < i1; b += 4) {
    float v[4][NP][4], f[4][NP];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = b + u < i1 ? b + u : b;
      const int64_t n = (int64_t)(uint32_t)ck[i];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int col = 256 * p + 4 * lane;
        if (col < W) {
          load4<Tv>(src + n * ld + col, v[u][p]);
          f[u][p] = gate ? gate[n * Hkv + col / hd] : 1.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (b + u >= i1) break;
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[p][e] = fmaf(f[u][p], v[u][p][e], acc[p][e]);
    }
  }
}

// One block (8 waves) per chunk of 64 sorted positions.  Runs of equal ids
// shorter than kLongRun go to the waves round-robin, each summed by one wave
// in sorted order; longer runs are split into 8 consecutive parts, one per
// wave, added pairwise in a fixed order through LDS.  (Eight waves: a run
// costs its wave a load round trip however short, and most runs of a Zipf
// batch are a row or two; 39 us per d12 table against 58 for four waves and
// 51 for sixteen.)  A run that is its id's whole
// segment is written as the final row; a run cut by the chunk's edge leaves a
// partial row (slot 0 if it starts the chunk, 1 if it ends it).
static constexpr int kLongRun = 16;
static constexpr int kSegWaves = 8;

template <int NP>
__device__ __forceinline__ void put_row(float* out, int W, int lane, bool add,
                                        const float (&acc)[NP][4]) {
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int col = 256 * p + 4 * lane;
    if (col < W) {
      float4 v = make_float4(acc[p][0], acc[p][1], acc[p][2], acc[p][3]);
      if (add) {
        const float4 q = *(const float4*)(out + col);
        v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
      }
      *(float4*)(out + col) = v;
    }
  }
}

template <typename Tv, int NP>
__global__ __launch_bounds__(64 * kSegWaves) void k_seg_rows(const uint64_t* keys, int64_t N,
                                                  const int32_t* first1, const int32_t* last1,
                                                  const Tv* src, int64_t ld, int W,
                                                  const float* gate, int Hkv, int hd,
                                                  float* dst, float* part, int accumulate) {
  static_assert(kChunk == 64, "one lane per chunk position");
  __shared__ uint64_t ck[kChunk];
  __shared__ float red[kSegWaves][NP * 256];
  const int64_t c0 = (int64_t)blockIdx.x * kChunk, c1 = std::min(N, c0 + kChunk);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int len = (int)(c1 - c0);
  if (threadIdx.x < kChunk) ck[threadIdx.x] = c0 + threadIdx.x < N ? keys[c0 + threadIdx.x] : kPad;
  __syncthreads();
  const bool start = lane < len && (lane == 0 || (ck[lane] >> 32) != (ck[lane - 1] >> 32));
  const uint64_t starts = __builtin_amdgcn_ballot_w64(start);
  // whole-segment flags of the runs, looked up once for the chunk
  __shared__ int wh[kChunk];
  if (w == 0 && start) {
    const uint32_t id = (uint32_t)(ck[lane] >> 32);
    const int64_t sf = first1[id] - 1, sl = last1[id];
    wh[lane] = sf >= c0 && sl <= c1;
  }
  __syncthreads();
  auto target = [&](int rs, int re, uint32_t id, bool* whole) {
    *whole = wh[rs] != 0;
    return *whole ? dst + (int64_t)id * W
                  : part + ((int64_t)blockIdx.x * 2 + (rs == 0 ? 0 : 1)) * W;
  };
  float acc[NP][4];
  // short runs: one wave each
  uint64_t m = starts;
  for (int r = 0; m; ++r) {
    const int rs = __builtin_ctzll(m);
    m &= m - 1;
    const int re = m ? __builtin_ctzll(m) : len;
    if (re - rs >= kLongRun || (r & (kSegWaves - 1)) != w) continue;
    const uint32_t id = (uint32_t)(ck[rs] >> 32);
    rows_sum<Tv, NP>(ck, rs, re, src, ld, W, gate, Hkv, hd, lane, acc);
    bool whole;
    float* out = target(rs, re, id, &whole);
    put_row<NP>(out, W, lane, whole && accumulate, acc);
  }
  // long runs: a quarter per wave
  m = starts;
  while (m) {
    const int rs = __builtin_ctzll(m);
    m &= m - 1;
    const int re = m ? __builtin_ctzll(m) : len;
    if (re - rs < kLongRun) continue;
    const int q = (re - rs + kSegWaves - 1) / kSegWaves;
    const int a = std::min(re, rs + w * q), b = std::min(re, a + q);
    rows_sum<Tv, NP>(ck, a, b, src, ld, W, gate, Hkv, hd, lane, acc);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][256 * p + 4 * lane + e] = acc[p][e];
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 256 * p + 4 * lane + e;
          float t[kSegWaves];                       // pairwise, fixed tree
#pragma unroll
          for (int k = 0; k < kSegWaves; ++k) t[k] = red[k][c];
#pragma unroll
          for (int n = kSegWaves / 2; n >= 1; n /= 2)
#pragma unroll
            for (int k = 0; k < n; ++k) t[k] = t[2 * k] + t[2 * k + 1];
          acc[p][e] = t[0];
        }
      const uint32_t id = (uint32_t)(ck[rs] >> 32);
      bool whole;
      float* out = target(rs, re, id, &whole);
      put_row<NP>(out, W, lane, whole && accumulate, acc);
    }
    __syncthreads();
  }
}

// One wavefront per id (4 ids per block): rows of absent ids are cleared
// (unless accumulating), ids cut by chunk boundaries get their partials added
// in chunk order.
__global__ __launch_bounds__(256) void k_seg_fix(const int32_t* first1, const int32_t* last1,
                                                 const float* part, int V, int W, float* dst,
                                                 int accumulate) {
  const int id = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (id >= V) return;
  const int32_t f1 = first1[id];
  float* out = dst + (int64_t)id * W;
  if (f1 == 0) {
    if (!accumulate)
      for (int col = 4 * lane; col < W; col += 256) *(float4*)(out + col) = make_float4(0, 0, 0, 0);
    return;
  }
  const int64_t sf = f1 - 1, se = last1[id];
  const int64_t ca = sf / kChunk, cb = (se - 1) / kChunk;
  if (ca == cb) return;                                 // written whole by k_seg_rows
  const int sa = sf == ca * kChunk ? 0 : 1;
  for (int col = 4 * lane; col < W; col += 256) {
    float4 v = *(const float4*)(part + (ca * 2 + sa) * W + col);
    for (int64_t c = ca + 1; c <= cb; c += 8) {         // 8 loads in flight, added in order
      float4 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        q[u] = c + u <= cb ? *(const float4*)(part + ((c + u) * 2) * W + col)
                           : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v.x += q[u].x; v.y += q[u].y; v.z += q[u].z; v.w += q[u].w;
      }
    }
    if (accumulate) {
      const float4 q = *(const float4*)(out + col);
      v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
    }
    *(float4*)(out + col) = v;
  }
}

hipError_t seg_scatter(const void* scratch, int64_t N, int V, int maxW, const void* src,
                       int64_t ld, int W, const float* gate, int Hkv, int hd, float* dst,
                       int accumulate, DType dt, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (W > 256 * kMaxPass || W % 4 || W > maxW) return hipErrorInvalidValue;
  const SortLayout L = sort_layout(N, V, maxW);
  const char* base = (const char*)scratch;
  const uint64_t* keys = (const uint64_t*)(base + L.keys[L.rounds & 1]);
  const int32_t* first1 = (const int32_t*)(base + L.first);
  const int32_t* last1 = (const int32_t*)(base + L.last);
  float* part = (float*)(base + L.part);
  const unsigned chunks = (unsigned)cdiv(N, kChunk);
  const int np = (int)cdiv(W, 256);
  const int es = dt == BF16 ? 2 : 4;
  const Work w(0.0, (double)N * (W * es + 12) + (double)V * W * 4 * (accumulate ? 2 : 1));
#define SEG_ROWS(TV, NPV)                                                                      \
  GK_LAUNCH(w, (k_seg_rows<TV, NPV>), dim3(chunks), dim3(64 * kSegWaves), 0, s, keys, N,       \
            first1, last1, (const TV*)src, ld, W, gate, Hkv, hd, dst, part, accumulate)
#define SEG_NP(TV)                                                                             \
  switch (np) {                                                                                \
    case 1: SEG_ROWS(TV, 1); break;                                                            \
    case 2: SEG_ROWS(TV, 2); break;                                                            \
    case 3: SEG_ROWS(TV, 3); break;                                                            \
    case 4: SEG_ROWS(TV, 4); break;                                                            \
    case 5: case 6: SEG_ROWS(TV, 6); break;                                                    \
    default: SEG_ROWS(TV, 8); break;                                                           \
  }
  if (dt == BF16) {
    SEG_NP(bf16)
  } else {
    SEG_NP(float)
  }
#undef SEG_NP
#undef SEG_ROWS
  GK_LAUNCH(Work(), k_seg_fix, dim3((unsigned)cdiv(V, 4)), dim3(256), 0, s, first1, last1,
            (const float*)part, V, W, dst, accumulate);
  return hipGetLastError();
}

}  // namespace gk
