// Host-side launchers of the gfx950 kernels (internal interface).
// Every launcher enqueues on `s` and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

enum DType { F32 = 0, BF16 = 1 };
enum GemmOp { OP_NT = 0, OP_NN = 1, OP_TN = 2 };
enum Epi { E_STORE = 0, E_RESADD, E_RELU2, E_DRELU2, E_F32, E_F32_ACC,
           E_CE,       // lm_ce_gemm only
           E_QKNORM,   // qkv_gemm_rope_norm only
           E_CEB };    // lm_ce_bwd_gemm only

// ---- elementwise / reductions -------------------------------------------
hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s);

hipError_t rope_table(float* cs, int T, int hd, float base, hipStream_t s);

// out [cols, rows] = in [rows, cols]^T, bf16, rows and cols multiples of 8
hipError_t transpose_bf16(const void* in, int64_t rows, int64_t cols, void* out, hipStream_t s);

// x[n, :] = wte[tok[b, t], :], n = b*T + t, tok rows of length T+1
hipError_t embed_fwd(const int32_t* tok, int B, int T, const void* wte,
                     void* x, int D, DType dt, hipStream_t s);
// dW[tok[n], :] += dx[n, :] (fp32)
hipError_t embed_bwd(const int32_t* tok, int B, int T, const void* dx,
                     int ldx, float* dW, int D, DType dt, hipStream_t s);

hipError_t rmsnorm_fwd(const void* x, void* y, float* r, int64_t rows, int D,
                       float eps, DType dt, hipStream_t s);
// x <- bf16(lam[0] x + lam[1] x0) stored to xout (may be x), then y = rms(x)
// (lam: 2 device bf16 values); bf16 rows, D % 8 == 0, D <= 2048 (else
// hipErrorInvalidValue: mix and norm run as two launches instead)
bool rmsnorm_fwd_mix_ok(int D, DType dt);
hipError_t rmsnorm_fwd_mix(const void* x, const void* x0, const void* lam, void* xout, void* y,
                           float* r, int64_t rows, int D, float eps, DType dt, hipStream_t s);
// dx = dres + r (g - y mean(g y)),  g = dy (+ VE term on the first C cols:
// sum_kv vez[n, kv] * wg[kv, c])
hipError_t rmsnorm_bwd(const void* dy, const void* y, const float* r,
                       const void* dres, void* dx, int64_t rows, int D,
                       const float* vez, const void* wg, int Hkv, int C,
                       DType dt, hipStream_t s);

struct GemmDesc {
  int op;            // GemmOp
  int64_t M, N, K;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  void* C; int64_t ldc;
  int epi;           // Epi
  void* aux;         // DRELU2: input a = relu(u)^2 (ldc, dtype)
  void* scratch;     // optional fp32 split-K partials (fp32 epilogues only)
  size_t scratch_bytes;
};
hipError_t gemm(const GemmDesc& g, DType dt, hipStream_t s);
// `batch` bf16 products of g's shape, A, B, C advanced by sa, sb, sc
// elements per product; E_STORE or E_F32, no aux, no K split.
hipError_t gemm_batched(const GemmDesc& g, int batch, int64_t sa, int64_t sb, int64_t sc,
                        hipStream_t s);
// scratch bytes gemm() would use for this bf16 product with an fp32 epilogue
size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K);

hipError_t rope_qknorm_fwd(void* qkv, float* rq, float* rk, const float* cs,
                           int B, int T, int H, int Hkv, int hd, float eps,
                           DType dt, hipStream_t s);
hipError_t rope_qknorm_bwd(void* dqkv, const void* qkv, const float* rq,
                           const float* rk, const float* cs, int B, int T,
                           int H, int Hkv, int hd, DType dt, hipStream_t s);

// value embedding: g[n,kv] = 3 sigmoid(h[n,:C] . wg[kv,:]); v += g * E[tok]
hipError_t ve_fwd(const int32_t* tok, int B, int T, const void* h, int D,
                  const void* wg, int C, const void* E, void* qkv, int ldqkv,
                  int voff, float* g, int Hkv, int hd, DType dt, hipStream_t s);
// vez[n,kv] = (sum_d dv e) g (1 - g/3);  dE[tok] += g dv
hipError_t ve_bwd(const int32_t* tok, int B, int T, const void* dqkv,
                  int ldqkv, int voff, const void* E, const float* g,
                  float* vez, float* dE, int Hkv, int hd, DType dt,
                  hipStream_t s);
// dWg[kv, c] (=/+=) sum_n vez[n, kv] h[n, c]; part: ve_wgrad_scratch_bytes
// of fp32 scratch (deterministic two-stage sum)
constexpr int kVeWgradBlocks = 512;
size_t ve_wgrad_scratch_bytes(int Hkv, int C);
hipError_t ve_wgrad(const float* vez, const void* h, int D, int64_t N,
                    int Hkv, int C, float* dWg, int accumulate, float* part,
                    DType dt, hipStream_t s);

// Token-sorted scatter into embedding-table gradients (deterministic):
// tok_sort orders the batch's ids once (scratch of tok_sort_bytes; maxW =
// the widest row later scattered), then seg_scatter sets (or adds to) dst[v,
// 0:W] the sum over positions n with token v of f(n, col) src[n*ld + col],
// f = gate[n*Hkv + col/hd] or 1.  W % 4 == 0, W <= 2048, ld % 4 == 0.
size_t tok_sort_bytes(int64_t N, int V, int maxW);
hipError_t tok_sort(const int32_t* tok, int B, int T, int V, int maxW, void* scratch,
                    hipStream_t s);
hipError_t seg_scatter(const void* scratch, int64_t N, int V, int maxW, const void* src,
                       int64_t ld, int W, const float* gate, int Hkv, int hd, float* dst,
                       int accumulate, DType dt, hipStream_t s);
// vez only (the value-embedding gate gradient), no table scatter
hipError_t ve_vez(const int32_t* tok, int B, int T, const void* dqkv, int ldqkv, int voff,
                  const void* E, const float* g, float* vez, int Hkv, int hd, DType dt,
                  hipStream_t s);

// score_bound > 0: the caller guarantees |q . k| / sqrt(hd) <= score_bound
// for every pair (QK-normed rows: sqrt(hd)); lets the kernel use one fixed
// softmax offset.  0: no bound known.
hipError_t attn_fwd(const void* qkv, void* o, float* lse, int B, int T,
                    int H, int Hkv, int hd, int W, DType dt, hipStream_t s,
                    float score_bound = 0.f);
size_t attn_bwd_scratch_bytes(int B, int T, int H, int hd);
// KV-cache decode attention (bf16, hd 128): q [B, Tq, H, 128], caches [B,
// Tmax, Hkv, 128], lens [B] (device, clamped to [0, Tmax]) -> o [B, Tq, H,
// 128], lse [B, H, Tq].  Query t of sequence b at position lens[b] - Tq + t.
// scratch: attn_decode_scratch_bytes (0: none needed).
size_t attn_decode_scratch_bytes(int B, int Tq, int H, int Hkv, int Tmax, int W);
// the leading part of that scratch that must be zero before a launch (the
// arrival counters; the kernel returns them to zero)
size_t attn_decode_counter_bytes(int B, int Tq, int H, int Hkv, int Tmax, int W);
hipError_t attn_decode(const void* q, const void* kc, const void* vc, const int32_t* lens,
                       void* o, float* lse, int B, int Tq, int Tmax, int H, int Hkv, int W,
                       float score_bound, void* scratch, hipStream_t s);
// With nrq / nrk / ncs (1/rms of the rotated q, k heads and the rope table)
// and attn_bwd_fuses_norm() true, the backward of RoPE-then-QK-norm is
// applied too (dq, dk w.r.t. the raw q, k); otherwise they are ignored.
bool attn_bwd_fuses_norm(int T, int H, int Hkv, int hd, DType dt);
// A second stream for work that may run beside s, with two events: `fork`
// (recorded on s, waited for by s2) and `join` (recorded on s2, waited for
// by s).  A null s2 means one stream.
struct Beside {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipStream_t s4 = nullptr;                    // optional: the dV pass there (else on s2)
  hipEvent_t join4 = nullptr;
};
hipError_t attn_bwd(const void* qkv, const void* o, const float* lse,
                    const void* dout, void* dqkv, void* scratch, int B, int T,
                    int H, int Hkv, int hd, int W, DType dt, hipStream_t s,
                    const float* nrq = nullptr, const float* nrk = nullptr,
                    const float* ncs = nullptr, const Beside& beside = Beside());

// cross-entropy over fp32 logits; tgt given by a token-row pointer:
// target of row n = tok[(n / T) * (T+1) + n % T + 1]  (T = tgt_T)
// (row0: token position of the first row, for chunked calls)
hipError_t ce_rows(const float* z, int64_t rows, int V, const int32_t* tok,
                   int tgt_T, int tgt_direct, float* ell, float* lse,
                   void* dz, float grad_scale, DType dt, hipStream_t s,
                   int64_t row0);
// loss = mean(ell[0:N]) (fp64 sum); flag = !isfinite(loss)
// QKV projection with RoPE then QK-norm fused into the product's epilogue
// (bf16, head_dim 128): qkv[rows, (H + 2 Hkv) 128] = h Wqkv^T, every q and k
// head rotated (position = row % T, table cs [T][64] (cos, sin)) and RMS-
// normalised, its 1/rms to rq [rows, H] / rk [rows, Hkv]; v heads stored as
// they are.  Same rounding points as gemm + rope_qknorm_fwd.
// With ve, the value embedding of a VE layer is applied to the v heads in the
// same epilogue: g = 3 sigmoid(h[:, :C] wg^T) per KV head (to ve->g [rows,
// Hkv]), v = v + g E[token] (token of row n: tok[(n / T)(T + 1) + n % T]).
struct VeArgs {
  const int32_t* tok;
  const void* wg;     // [Hkv, C]
  int C;
  const void* E;      // [V, Hkv hd]
  float* g;
};
bool qkv_rope_fused_ok(int64_t rows, int D, int H, int Hkv, int hd);
hipError_t qkv_gemm_rope_norm(const void* h, int64_t rows, int D, const void* wqkv, int H,
                              int Hkv, void* qkv, const float* cs, float* rq, float* rk, int T,
                              float eps, const VeArgs* ve, hipStream_t s);
// Fused lm_head + cross-entropy for bf16 (V a multiple of 256, products the
// direct-to-LDS GEMM takes).  lm_ce_gemm: logits = hf[rows, D] Wlm[V, D]^T,
// never stored as such; per row and 256-column tile t the max m_t of the
// logits and s_t = sum exp(logit - m_t) go to stats[row * (V / 256) + t],
// the target's logit to zt[row], and (if e) e = exp(logit - m_t) as bf16 to
// e[row * V + col].  ce_fix: with ell (and zt), lse = max_t m_t +
// log(sum_t s_t exp(m_t - max)) and ell = lse - zt go out; with dz, dz =
// (e exp(m_t - lse) - onehot) * grad_scale as bf16 (dz may be e itself),
// from the lse just formed or, without ell, the one lse holds.  Targets as
// in ce_rows.
bool lm_ce_fused_ok(int64_t rows, int V, int D);
size_t lm_ce_stats_bytes(int64_t rows, int V);
// (tgt_direct: the target of row n is tok[n] instead)
hipError_t lm_ce_gemm(const void* hf, int64_t rows, int D, const void* wlm, int V, void* e,
                      float* stats, float* zt, const int32_t* tok, int tgt_T, int tgt_direct,
                      hipStream_t s);
hipError_t ce_fix(const float* stats, const float* zt, int64_t rows, int V, const int32_t* tok,
                  int tgt_T, int tgt_direct, float* ell, float* lse, const void* e, void* dz,
                  float grad_scale, hipStream_t s);
// The lm_head's input gradient straight from lm_ce_gemm's e:
// dh[rows, D] = dz Wlm with dz = (e exp(m_t - lse) - onehot) * grad_scale,
// without forming dz.  The product runs over the vocabulary in 256-column
// tiles with the accumulator kept in units of the current tile's exp(m_t)
// (rescaled at each tile boundary), the final scale and the target's row of
// Wlm applied in the epilogue.
bool lm_ce_bwd_ok(int64_t rows, int V, int D);
hipError_t lm_ce_bwd_gemm(const void* e, int64_t rows, int V, const void* wlm, int D, void* dh,
                          const float* stats, const float* lse, const int32_t* tok, int tgt_T,
                          int tgt_direct, float grad_scale, hipStream_t s);
// FP8 linear layers with tensor-wise scaling.  fp8_cast: q = fp8(clamp(x s,
// +-fmax)), s = fmax / max(max|x|, 1e-12), x [rows, cols] (cols % 16 == 0;
// rows % 16 == 0 when qt is given), row-major into q and/or transposed into
// qt ([cols, rows]); scales[0] = s, scales[1] = 1/s.  fmt 0: e4m3, 1: e5m2.
// scratch: fp8_cast_scratch_bytes.
size_t fp8_cast_scratch_bytes();
hipError_t fp8_cast(const void* x, int64_t rows, int64_t cols, DType dt, int fmt, void* q,
                    void* qt, float* scales, void* scratch, hipStream_t s);
// gemm_fp8: C[M, N] = (A[M, K] B[N, K]^T) a_inv[0] b_inv[0], K-contiguous
// fp8 operands (formats fa, fb), epi E_STORE (bf16), E_F32 or E_F32_ACC;
// scratch: split-K partials (gemm_fp8_scratch_bytes for the full split).
bool gemm_fp8_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc);
size_t gemm_fp8_scratch_bytes(int64_t M, int64_t N, int64_t K);
hipError_t gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                    const void* B, int64_t ldb, int fb, const float* a_inv, const float* b_inv,
                    void* C, int64_t ldc, int epi, void* scratch, size_t scratch_bytes,
                    hipStream_t s);
// Muon's Newton-Schulz orthogonalization of `batch` matrices G [m, n]
// (dtype, contiguous): X =
// G / (||G||_F + eps), then per tuple (a, b, c) of coeffs (host, 3 steps
// floats) X <- X (a I + b A + c A A), A = X^T X (tall) or the transposed
// form (wide); result bf16 in x_out [m, n]; ws: polar_express_ws_bytes.
size_t polar_express_ws_bytes(int batch, int64_t m, int64_t n);
hipError_t polar_express(const void* g, int batch, int64_t m, int64_t n, DType dt,
                         const float* coeffs, int steps, float eps, void* x_out, void* ws,
                         hipStream_t s);
// Optimizer elementwise steps (n a multiple of 4, 16-byte aligned):
// Muon momentum M <- beta M + (1 - beta) G, U = Nesterov look-ahead or M;
// Muon step W <- W (1 - lr wd) - lr X (X bf16); AdamW (step counts from 1).
// w16: optional bf16 copy of the updated weights.
hipError_t muon_momentum(const float* g, float* mom, void* u, int64_t n, float beta, int nesterov,
                         DType u_dt, hipStream_t s);
hipError_t muon_update(float* w, const void* x, int64_t n, float lr, float wd, void* w16,
                       hipStream_t s);
hipError_t adamw(float* w, const float* g, float* m, float* v, int64_t n, int step, float lr,
                 float b1, float b2, float eps, float wd, void* w16, hipStream_t s);
// muon_momentum / muon_update over the equally shaped matrices of a group
// (1 <= layers <= kMaxGroupLayers) in one launch: matrix y's fp32 tensors at
// element offset offs.off[y] of g / mom / w (and w16), its u / x at slot y
// of a contiguous [layers, n] buffer; n a multiple of 4
constexpr int kMaxGroupLayers = 64;
struct LayerOffsets { int64_t off[kMaxGroupLayers]; };
hipError_t muon_momentum_group(const float* g, float* mom, void* u, const LayerOffsets& offs,
                               int layers, int64_t n, float beta, int nesterov, DType u_dt,
                               hipStream_t s);
hipError_t muon_update_group(float* w, const void* x, const LayerOffsets& offs, int layers,
                             int64_t n, float lr, float wd, void* w16, hipStream_t s);
// NorMuon variant of muon_update_group on matrices [rows, cols] (cols a
// multiple of 8): per row the mean square of X's row updates the second
// moment v (matrix y's at v + offs.off[y], `rows` floats), then W <- W (1 -
// lr wd) - lr f_r X with f_r = v_r^(-1/2) ||X||_F / ||v^(-1/2) X||_F (the
// floor 1e-10 under v and the norm); scratch: normuon_scratch_bytes.
size_t normuon_scratch_bytes(int layers, int64_t rows);
hipError_t normuon_update_group(float* w, const void* x, float* v, const LayerOffsets& offs,
                                int layers, int64_t rows, int64_t cols, float b2, float lr,
                                float wd, void* w16, void* scratch, hipStream_t s);
// Number of ids outside [0, V) among tok[0 .. n) written to *count (one
// workgroup, fixed order).
hipError_t count_bad_ids(const int32_t* tok, int64_t n, int V, int* count, hipStream_t s);
// Model extras.  resid_mix: y = lr x + l0 x0 with (lr, l0) by `mode`:
// MIX_LAMBDAS (lam[0], lam[1]), lam 2 device values of the storage type;
// MIX_BACKOUT (1, -lam[0]); MIX_ADD (1, 1).  y may be x.  Backward dx = lr dy (dx may be null or dy), dx0 (+)= l0 dy,
// dlam (=, or += with accumulate_dlam): MIX_LAMBDAS [0..2) = sums of dy x,
// dy x0; MIX_BACKOUT [0] = -sum dy x0 (x unused).
// smear: y_t = x_t + g_t x_(t-1), g_t = lam[0] sigmoid(w . x_t[:24]),
// g_t = 0 at a row's first position (rows of T tokens); backward dx (not
// dy) and dw_dlam[0..24) = dw, [24] = dlambda (= or +=).  n, D multiples
// of 8.
enum { MIX_LAMBDAS = 0, MIX_BACKOUT = 1, MIX_ADD = 2 };
// p[0..n) = 0 for fp32 at any 4-byte alignment (a kernel, not a memset)
hipError_t zero_f32(float* p, int64_t n, hipStream_t s);
size_t resid_mix_bwd_scratch_bytes();
size_t smear_bwd_scratch_bytes();
hipError_t resid_mix_fwd(const void* x, const void* x0, void* y, int64_t n, const void* lam,
                         DType dt, hipStream_t s, int mode = MIX_LAMBDAS);
hipError_t resid_mix_bwd(const void* dy, const void* x, const void* x0, void* dx, void* dx0,
                         int accumulate, int64_t n, const void* lam, float* dlam, void* scratch,
                         DType dt, hipStream_t s, int mode = MIX_LAMBDAS,
                         int accumulate_dlam = 0);
hipError_t smear_fwd(const void* x, int64_t rows, int T, int D, const void* w, const void* lam,
                     void* y, float* gate, DType dt, hipStream_t s);
hipError_t smear_bwd(const void* dy, const void* x, int64_t rows, int T, int D, const void* w,
                     const void* lam, const float* gate, void* dx, float* dw_dlam,
                     void* scratch, DType dt, hipStream_t s, int accumulate_dw = 0);
hipError_t loss_reduce(const float* ell, int64_t N, float* loss_ws,
                       float* loss_out, int* flag, hipStream_t s);
// acc[0] += sum ell, acc[1] += sum bytes[tgt]; if final, acc[2] = bpb
hipError_t eval_accum(const float* ell, const int32_t* tok, int rows, int T,
                      const int32_t* token_bytes, double* acc, int first,
                      hipStream_t s);
hipError_t eval_finish(const double* acc, double* out, hipStream_t s);

}  // namespace gk
