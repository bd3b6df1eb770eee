/*
 * gpt_step.h -- C ABI of the MI355X (gfx950) GPT training-step library.
 *
 * The library computes one forward + backward training step of the compact
 * GPT decoder described by the nanochat walkthrough ("5만원으로 나만의 ChatGPT
 * 훈련하는 방법", apidog.com, section "1. GPT model (nanochat/gpt.py)":
 * rotary embeddings, QK normalisation, untied weights, ReLU^2 MLP, grouped-
 * query attention, sliding-window pattern, value embeddings with a per-head
 * gate) and scores it in bits per byte (tilnote.io autoresearch summary,
 * "core mechanism": val_bpb).  Normalisation is RMSNorm with residual
 * connections ("microgpt", news.hada.io, "model architecture"); the loss is
 * the next-token cross-entropy ("microgpt", "training loop").
 *
 * Conventions for every entry point
 *   - Pointers named *_dev or documented as "device" are device memory owned
 *     by the caller and must stay valid until the enqueued work completes.
 *     They must be 16-byte aligned (GPT_ERR_MISALIGNED otherwise).
 *   - Work is enqueued on the caller's stream; no call synchronises the host.
 *   - The library allocates no device memory: all scratch lives in the
 *     caller's workspace `ws` (size from gpt_workspace_bytes).
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     negative return means nothing was enqueued; gpt_last_error() then holds
 *     a message (thread-local).  Asynchronous device faults surface at the
 *     caller's next stream synchronisation.
 *   - Calls with distinct workspaces may run concurrently on distinct streams.
 */
#ifndef GPT_STEP_H
#define GPT_STEP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  GPT_OK = 0,
  GPT_ERR_INVALID_ARG = -1,        /* null pointer, bad size or flag        */
  GPT_ERR_UNSUPPORTED_CONFIG = -2, /* config outside what the kernels cover */
  GPT_ERR_WORKSPACE_TOO_SMALL = -3,
  GPT_ERR_MISALIGNED = -4,         /* a pointer is not 16-byte aligned      */
  GPT_ERR_HIP = -5                 /* a HIP runtime call failed             */
};

/* storage dtype of parameters and activations */
enum { GPT_F32 = 0, GPT_BF16 = 1 };

/* workspace modes */
enum { GPT_MODE_TRAIN = 0, GPT_MODE_EVAL = 1 };

/*
 * Model configuration.
 *   n_layer, d_model (D), n_head (H), n_kv_head (Hkv, divides H), head_dim
 *   (hd: 4, 8, 16, 32, 64 or 128), vocab (V), seq_len (T), batch (B rows),
 *   mlp_mult (MLP width F = mlp_mult * D), ve_gate_channels (C: the value-
 *   embedding gate reads the first C channels of the normalised attention
 *   input, 1 <= C <= D).
 *   window_pattern: "" = full causal in every layer; otherwise characters
 *   'S'/'L', layer l uses pattern[l % len] -> window_short / window_long.
 *   Key j is visible from query i iff 0 <= i - j <= window (the window counts
 *   keys to the left of the query, as the window_size argument of the
 *   nanochat walkthrough's flash-attention call, section "5").
 *   ve_every_odd: 1 = value embeddings on layers 1, 3, 5, ... (0-based).
 *   rope_base: rotary base; theta_{t,j} = t * base^(-2j/hd), pairs (j, j+hd/2).
 *   norm_eps: added to the mean square inside every RMSNorm root.
 *   dtype: GPT_BF16 (bf16 storage, fp32 accumulation, fp32 softmax/CE) or
 *   GPT_F32 (fp32 storage).
 *   Model extras (nanochat walkthrough, "1. GPT model", efficiency tricks),
 *   each off when 0 (a zero-filled tail keeps the plain model):
 *   resid_lambdas: 1 = before block l the stream becomes lr_l x + l0_l x0,
 *     x0 the stream the blocks start from.
 *   smear: 1 = right after the embedding, x_t += g_t x_(t-1) with g_t =
 *     lambda_s sigmoid(w_s . x_t[:24]), g = 0 at a row's first position
 *     (needs D >= 24).
 *   backout: 1 = the stream after block backout_layer (0 <= it < n_layer)
 *     is kept and, after the last block, x -= lambda_b x_kept.
 *   With any extra on, D must be a multiple of 8.
 *   check_tokens: 1 = gpt_step_fwd, gpt_step_bwd and gpt_eval_bpb first
 *     count the token ids outside [0, V) on the device, wait for the count
 *     (a stream synchronisation) and return GPT_ERR_INVALID_ARG, with the
 *     count in gpt_last_error(), when it is not zero; nothing but that
 *     check has been enqueued then.  0 = ids are a precondition (no check,
 *     no synchronisation).  A library built for debugging
 *     (`python -m gpt_pretraining_step_amd.build --debug`) checks always.
 *   one_stream: 1 = gpt_step_bwd runs everything on the caller's stream.
 *     0 = for bf16 models of at least 4096 tokens the weight-gradient
 *     products and the embedding and gate gradients run on a second,
 *     library-owned stream, and (head_dim 128) the attention backward's dQ
 *     and dV passes on two more (all per host thread and device, default
 *     priority), forked from and joined back into the caller's stream with
 *     events, so the call still completes in the caller's stream order (and
 *     can be captured into a graph).  Beside the caller's stream the linear
 *     layers' weight-gradient products split K at most 4 ways, so those
 *     four gradients differ from the one-stream results by fp32 summation
 *     order; every other result is bit for bit the same, and each mode is
 *     deterministic.
 */
typedef struct gpt_config {
  int32_t n_layer, d_model, n_head, n_kv_head, head_dim, vocab, seq_len, batch;
  int32_t mlp_mult, ve_gate_channels;
  char window_pattern[16];
  int32_t window_short, window_long;
  int32_t ve_every_odd;
  float rope_base, norm_eps;
  int32_t dtype;
  int32_t resid_lambdas, smear, backout, backout_layer;
  int32_t check_tokens;
  int32_t one_stream;
} gpt_config;

/* ------------------------------------------------------- sizes and layout */
/*
 * Flat parameter buffer, in this order, every matrix [out, in] row-major
 * (the weight of F.linear, nanochat walkthrough section "3. precision
 * management"):
 *   wte [V, D]
 *   per layer l: Wqkv [(H + 2 Hkv) hd, D] (rows: q heads, k heads, v heads),
 *                Wo [D, H hd], Wfc [F, D], Wproj [D, F],
 *                and on value-embedding layers E_l [V, Hkv hd], Wg [Hkv, C]
 *   Wlm [V, D]
 *   extras [8 ceil((2 L + 26) / 8)], only when a model extra is on: lr_l at
 *     2 l, l0_l at 2 l + 1, w_s at 2 L .. 2 L + 23, lambda_s at 2 L + 24,
 *     lambda_b at 2 L + 25, zero padding after (slots of extras that are
 *     off are unused, their gradients zero)
 * Gradients use the same layout in fp32.
 */
enum {
  GPT_P_WTE = 0, GPT_P_WQKV, GPT_P_WO, GPT_P_WFC, GPT_P_WPROJ, GPT_P_VE,
  GPT_P_WG, GPT_P_WLM, GPT_P_EXTRAS
};

/* Number of parameters (elements), or a negative status for a bad config. */
int64_t gpt_param_count(const gpt_config* cfg);

/* Element offset of tensor `which` (GPT_P_*) of `layer` in the flat buffer;
 * -1 if that layer has no such tensor; a status < -1 for a bad argument.
 * `layer` is ignored for GPT_P_WTE, GPT_P_WLM and GPT_P_EXTRAS (-1 when no
 * extra is on). */
int64_t gpt_param_offset(const gpt_config* cfg, int which, int layer);

/* Workspace bytes needed by gpt_step_fwd/bwd (GPT_MODE_TRAIN) or by
 * gpt_eval_bpb (GPT_MODE_EVAL); 0 for a bad config (see gpt_last_error). */
size_t gpt_workspace_bytes(const gpt_config* cfg, int mode);

/* Check a config without touching the GPU; returns a status. */
int gpt_validate_config(const gpt_config* cfg);

/* --------------------------------------------------------------- the step */
/*
 * Forward pass and mean next-token cross-entropy of one batch.
 *   params : device, dtype per cfg->dtype, the flat layout above.
 *   tokens : device int32 [B, T+1] row-major; inputs are the first T ids of a
 *            row, targets the last T.  Ids outside [0, V) are a precondition
 *            violation, checked only with cfg->check_tokens (or in a debug
 *            build): then GPT_ERR_INVALID_ARG before any gather runs.
 *   ws     : device workspace of ws_bytes >= gpt_workspace_bytes(TRAIN).  The
 *            forward saves what the backward needs in it; ws[] also holds the
 *            per-token losses (gpt_ws_offset(GPT_WS_ELL)).
 *   loss_dev : device float, receives mean loss over the B*T targets.
 * Softmax and cross-entropy are fp32; logits are fp32.  What the backward
 * needs of the softmax gradient (softmax - onehot)/(B T) stays in ws: for
 * bf16 models with V a multiple of 256, exp(logit - max) per 256-column
 * tile (bf16) with each tile's max and the row's lse, from which the
 * backward forms the gradient itself; otherwise the gradient (dtype).  A
 * non-finite loss sets the int32 flag at GPT_WS_NONFINITE.
 */
int gpt_step_fwd(const gpt_config* cfg, const void* params,
                 const int32_t* tokens, void* ws, size_t ws_bytes,
                 float* loss_dev, hipStream_t stream);

/*
 * Backward pass of the preceding gpt_step_fwd on the same ws, params and
 * tokens (upstream gradient of the mean loss = 1).
 *   grads : device fp32, flat layout; overwritten (accumulate = 0) or added
 *           to (accumulate = 1, for gradient accumulation over micro-batches).
 */
int gpt_step_bwd(const gpt_config* cfg, const void* params,
                 const int32_t* tokens, void* ws, size_t ws_bytes,
                 float* grads, int accumulate, hipStream_t stream);

/*
 * Bits per byte over an evaluation set (forward only).
 *   tokens      : device int32 [n_rows, T+1]; rows are processed in batches
 *                 of cfg->batch rows (the last one may be shorter); n_rows
 *                 >= 1 (an empty set is GPT_ERR_INVALID_ARG, nothing is
 *                 enqueued).
 *   token_bytes : device int32 [V], UTF-8 byte length of each vocabulary id,
 *                 indexed by the target id.
 *   ws          : ws_bytes >= gpt_workspace_bytes(EVAL).
 *   out_dev     : device double[3] = { sum of nats, sum of bytes,
 *                 bpb = nats / (ln 2 * bytes) }.
 */
int gpt_eval_bpb(const gpt_config* cfg, const void* params,
                 const int32_t* tokens, int64_t n_rows,
                 const int32_t* token_bytes, void* ws, size_t ws_bytes,
                 double* out_dev, hipStream_t stream);

/* ------------------------------------------------------ optimizer step */
/*
 * One optimizer step over the flat parameter layout (the nanochat
 * walkthrough, section "2. Muon optimizer": Muon for the block matrices,
 * AdamW for embeddings, lm_head and value embeddings).
 *   Muon, per block matrix [rows, cols] (Wqkv, Wo, Wfc, Wproj): momentum
 *   (state1) M <- mu M + (1 - mu) G, update U = (1 - mu) G + mu M
 *   (Nesterov) or M; X = the Newton-Schulz orthogonalization of U (ns_steps
 *   tuples from ns_coeffs, the same matrix of every layer batched);
 *   W <- W (1 - lr wd) - lr X with lr = muon_lr max(1, rows / cols)^0.5.
 *   NorMuon (normuon != 0; the same section's per-neuron normalisation):
 *   X is rescaled per output row before the step, X_r <- X_r s_r
 *   ||X||_F / ||diag(s) X||_F with s_r = 1 / sqrt(max(v_r, 1e-10)) and
 *   v_r <- normuon_beta2 v_r + (1 - normuon_beta2) mean_c X[r, c]^2 kept
 *   in state2 (its first `rows` floats in each Muon matrix's slot; zero
 *   before step 1); the second norm is clamped below at 1e-10.
 *   AdamW (state1 = m, state2 = v, step counts from 1): wte and the value-
 *   embedding tables at adam_lr_embed, Wlm at adam_lr_head, the value-
 *   embedding gates and the extras vector (the model extras' scalars and
 *   smear weights, when present) at adam_lr_gate.
 *   master, grads, state1, state2: device fp32 in the flat layout (states
 *   zero before step 1).  params: the dtype copy the step reads, written
 *   from the updated master (bf16 configs; may be null for fp32 configs,
 *   whose master is the parameter buffer).  ws: gpt_optim_ws_bytes(cfg)
 *   (one region per Muon group).  For bf16 configs without one_stream, the
 *   Muon groups other than the first run on the library's side streams,
 *   forked from and joined back into `stream` with events, so the call
 *   completes in `stream` order; results do not depend on it.
 *   Tensor offsets must be multiples of 8 elements (true when D, F, the
 *   qkv width and H hd are). */
typedef struct gpt_optim_hparams {
  float muon_lr, muon_momentum, muon_wd;
  int32_t muon_nesterov, ns_steps;  /* ns_steps <= 16 */
  float ns_coeffs[48];              /* (a, b, c) per step */
  float ns_eps;
  float adam_lr_embed, adam_lr_head, adam_lr_gate;
  float adam_beta1, adam_beta2, adam_eps, adam_wd;
  int32_t normuon;                  /* 0: plain Muon (a zeroed tail keeps it) */
  float normuon_beta2;              /* second-moment decay, [0, 1) */
} gpt_optim_hparams;

size_t gpt_optim_ws_bytes(const gpt_config* cfg);
int gpt_optim_step(const gpt_config* cfg, const gpt_optim_hparams* hp,
                   int32_t step, float* master, void* params,
                   const float* grads, float* state1, float* state2, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------- workspace inspection */
/* Byte offset into a TRAIN workspace of a saved tensor, for tests and
 * debugging; -1 when absent.  Layer-wise items take `layer`. */
enum {
  GPT_WS_ELL = 0,       /* fp32 [B*T] per-token loss                         */
  GPT_WS_LOSS,          /* fp32 scalar mean loss                             */
  GPT_WS_NONFINITE,     /* int32 flag, 1 if the loss was not finite          */
  GPT_WS_X_H,           /* dtype [N, D] normalised attention input  (layer)  */
  GPT_WS_X_QKV,         /* dtype [N, (H+2Hkv) hd] q,k after rotary+norm,
                           v after value embedding                  (layer)  */
  GPT_WS_X_O,           /* dtype [N, H hd] attention output          (layer)  */
  GPT_WS_X_LSE,         /* fp32 [B, H, T] attention log-sum-exp      (layer)  */
  GPT_WS_X_H2,          /* dtype [N, D] normalised MLP input         (layer)  */
  GPT_WS_X_A,           /* dtype [N, F] relu(u)^2                    (layer)  */
  GPT_WS_X_HF,          /* dtype [N, D] final normalised features            */
  GPT_WS_BAD_TOKENS     /* int32, ids outside [0, V) at the last check       */
};
int64_t gpt_ws_offset(const gpt_config* cfg, int which, int layer);

/* ------------------------------------------------------------- errors */
const char* gpt_status_string(int status);
const char* gpt_last_error(void);

/* ------------------------------------------------ kernel-level entries */
/*
 * Single kernels of the step, for parity tests and profiling.  Same
 * conventions; `dtype` (GPT_F32/GPT_BF16) is the storage type of the
 * activation arguments.  Statistics (r, lse) are fp32.
 */

/* y = x / sqrt(mean(x^2) + eps) per row of x [rows, dim]; r[row] = 1/sqrt(.) */
int gpt_k_rmsnorm_fwd(const void* x, void* y, float* r, int64_t rows,
                      int32_t dim, float eps, int32_t dtype, hipStream_t s);

/* dx = dres + r (dy - y mean(dy y)); dres may be null (= 0), dx may alias
 * dres.  All [rows, dim]. */
int gpt_k_rmsnorm_bwd(const void* dy, const void* y, const float* r,
                      const void* dres, void* dx, int64_t rows, int32_t dim,
                      int32_t dtype, hipStream_t s);

/*
 * C = op(A, B) over M x N x K with fp32 accumulation.
 *   op GPT_GEMM_NT: A [M, K] (lda), B [N, K] (ldb):   C = A B^T   (y = x W^T)
 *   op GPT_GEMM_NN: A [M, K] (lda), B [K, N] (ldb):   C = A B     (dx = dy W)
 *   op GPT_GEMM_TN: A [K, M] (lda), B [K, N] (ldb):   C = A^T B   (dW = dy^T x)
 *   epilogue GPT_EPI_STORE   : C (dtype) = acc
 *            GPT_EPI_RESADD  : C (dtype) = C + acc, rounded once
 *            GPT_EPI_RELU2   : C (dtype) = relu(u)^2, u = acc rounded to dtype
 *                              (aux ignored for every epilogue but DRELU2)
 *            GPT_EPI_DRELU2  : C (dtype) = acc * 2 sqrt(aux), aux (dtype, ldc)
 *                              holding a = relu(u)^2 as RELU2 wrote it, so
 *                              sqrt(aux) stands for relu(u)
 *            GPT_EPI_F32     : C (fp32) = acc
 *            GPT_EPI_F32_ACC : C (fp32) += acc
 */
enum { GPT_GEMM_NT = 0, GPT_GEMM_NN = 1, GPT_GEMM_TN = 2 };
enum { GPT_EPI_STORE = 0, GPT_EPI_RESADD, GPT_EPI_RELU2, GPT_EPI_DRELU2,
       GPT_EPI_F32, GPT_EPI_F32_ACC };
/* scratch (may be null): device fp32 space for split-K partial tiles of
 * fp32-epilogue bf16 products; gpt_k_gemm_scratch_bytes gives the size that
 * lets the product split as far as it wants (less scratch, fewer splits).
 * The result does not depend on whether or how the product is split, up to
 * fp32 summation order. */
size_t gpt_k_gemm_scratch_bytes(int64_t M, int64_t N, int64_t K);
int gpt_k_gemm(int32_t op, int64_t M, int64_t N, int64_t K, const void* A,
               int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
               int32_t epilogue, void* aux, void* scratch, size_t scratch_bytes,
               int32_t dtype, hipStream_t s);

/* FP8 linear layers with tensor-wise scaling (the nanochat walkthrough,
 * section "3. precision management": with --fp8 most linear layers become
 * Float8Linear with tensor-wise scales).  Formats are the OCP 8-bit floats:
 * GPT_FP8_E4M3 (max 448; activations and weights) and GPT_FP8_E5M2 (max
 * 57344; gradients). */
enum { GPT_FP8_E4M3 = 0, GPT_FP8_E5M2 = 1 };

/* Cast x [rows, cols] (dtype, device) with its tensor-wise scale:
 * s = fmax / max(max |x|, 1e-12) (fp32), q = fp8(clamp(x * s, -fmax, fmax))
 * rounded to nearest even (NaN stays NaN).  Outputs (device, 16-byte
 * aligned, either may be null but not both): q [rows, cols] row-major and
 * q_t [cols, rows] (its transpose, for the products that contract over
 * rows); scales[0] = s, scales[1] = 1/s (device fp32, 4-byte aligned).
 * Needs cols a
 * multiple of 16, and rows too when q_t is given.  scratch: device, >=
 * gpt_k_fp8_cast_scratch_bytes() bytes (per-block maxima). */
size_t gpt_k_fp8_cast_scratch_bytes(void);
int gpt_k_fp8_cast(const void* x, int64_t rows, int64_t cols, int32_t dtype,
                   int32_t fp8_format, void* q, void* q_t, float* scales,
                   void* scratch, size_t scratch_bytes, hipStream_t s);

/* FP8 product: C [M, N] = (A [M, K] . B [N, K]^T) * a_inv_scale[0] *
 * b_inv_scale[0], both operands K-contiguous 8-bit floats of the given
 * formats (leading dimensions lda, ldb in bytes), fp32 accumulation.
 * epilogue GPT_EPI_STORE (C bf16), GPT_EPI_F32 (C fp32) or GPT_EPI_F32_ACC
 * (C fp32 +=).  For y = x W^T pass A = q(x), B = q(W); for dX = dY W pass
 * A = q(dY), B = q_t(W); for dW = dY^T X pass A = q_t(dY), B = q_t(X).
 * Needs K a multiple of 128, lda and ldb multiples of 16 and >= K, N and
 * ldc multiples of 4, each operand under 4 GiB.  scratch (optional, fp32
 * outputs): split-K partials, up to gpt_k_gemm_fp8_scratch_bytes(M, N, K)
 * bytes; the product splits K only as far as the scratch allows. */
size_t gpt_k_gemm_fp8_scratch_bytes(int64_t M, int64_t N, int64_t K);
int gpt_k_gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, int32_t fmt_a, const void* B, int64_t ldb,
                   int32_t fmt_b, const float* a_inv_scale,
                   const float* b_inv_scale, void* C, int64_t ldc,
                   int32_t epilogue, void* scratch, size_t scratch_bytes,
                   hipStream_t s);

/* Muon's orthogonalization of matrix updates (the nanochat walkthrough,
 * section "2. Muon optimizer": quintic Newton-Schulz, "Polar Express").
 *   g [batch, m, n] (dtype, device, contiguous): `batch` updates of one
 *   shape (e.g. the same parameter of every layer), each orthogonalized on
 *   its own; they share the launches.
 *   coeffs (host): steps tuples (a, b, c), 3 * steps floats; the page
 *   prints the first two of its five tuples, so the caller supplies them.
 *   X = g / (||g||_F + eps); each tuple (a, b, c) replaces X by its odd
 *   quintic a X + b X (X^T X) + c X (X^T X)^2, formed as X (a I + b A +
 *   c A A) with A = X^T X (a matrix with fewer rows than columns takes
 *   A = X X^T and X <- (a I + b A + c A A) X).  X, A and the polynomial
 *   matrix are bf16 between the products (fp32 accumulation).
 *   x_out [batch, m, n] bf16 (device).  ws: device, >=
 *   gpt_k_polar_express_ws_bytes(batch, m, n).  Needs m and n multiples of
 *   8, 1 <= batch <= 65535, 0 <= steps <= 64.  Deterministic. */
size_t gpt_k_polar_express_ws_bytes(int32_t batch, int64_t m, int64_t n);
int gpt_k_polar_express(const void* g, int32_t batch, int64_t m, int64_t n,
                        int32_t dtype, const float* coeffs, int32_t steps,
                        float eps, void* x_out, void* ws, size_t ws_bytes,
                        hipStream_t s);

/* The elementwise parts of the optimizer step (the nanochat walkthrough,
 * section "2. Muon optimizer": Muon for the block matrices, AdamW for
 * embeddings, lm_head and value embeddings).  All buffers device, 16-byte
 * aligned, n elements (a multiple of 4); fp32 master weights, w_bf16 an
 * optional bf16 copy of the updated weights (the step's parameters).
 *   gpt_k_muon_momentum: mom <- beta mom + (1 - beta) grad, then
 *     u = (1 - beta) grad + beta mom (Nesterov) or mom, as u_dtype (the
 *     input of gpt_k_polar_express).
 *   gpt_k_muon_update: w <- w (1 - lr wd) - lr x, x the orthogonalized
 *     update (bf16); lr carries any shape factor.
 *   gpt_k_adamw: m <- b1 m + (1 - b1) g, v <- b2 v + (1 - b2) g^2,
 *     w <- w (1 - lr wd) - lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step))
 *     + eps); step counts from 1. */
int gpt_k_muon_momentum(const float* grad, float* mom, void* u, int64_t n,
                        float beta, int32_t nesterov, int32_t u_dtype,
                        hipStream_t s);
int gpt_k_muon_update(float* w, const void* x, int64_t n, float lr, float wd,
                      void* w_bf16, hipStream_t s);
/* NorMuon's step on one matrix (the nanochat walkthrough, section "2. Muon
 * optimizer", the per-neuron normalisation after the orthogonalization):
 * x [rows, cols] bf16 the orthogonalized update, v [rows] fp32 the per-row
 * second moment (in/out, zero before the first step), w [rows, cols] fp32
 * (in/out), w_bf16 an optional bf16 copy.  m_r = mean_c x[r, c]^2,
 * v_r <- beta2 v_r + (1 - beta2) m_r, s_r = 1 / sqrt(max(v_r, 1e-10)),
 * f_r = s_r sqrt(sum_r m_r) / max(sqrt(sum_r m_r s_r^2), 1e-10), then
 * w <- w (1 - lr wd) - lr f_r x.  cols a multiple of 8, rows cols < 2^31.
 * scratch: device, >= gpt_k_normuon_scratch_bytes(rows).  Deterministic
 * (fixed-order sums). */
size_t gpt_k_normuon_scratch_bytes(int64_t rows);
int gpt_k_normuon_update(float* w, const void* x, float* v, int64_t rows,
                         int64_t cols, float beta2, float lr, float wd,
                         void* w_bf16, void* scratch, size_t scratch_bytes,
                         hipStream_t s);
int gpt_k_adamw(float* w, const float* grad, float* m, float* v, int64_t n,
                int32_t step, float lr, float beta1, float beta2, float eps,
                float wd, void* w_bf16, hipStream_t s);

/* Model extras (the nanochat walkthrough, section "1. GPT model
 * (nanochat/gpt.py)", efficiency tricks).  Token-major rows [N, D] of
 * `dtype`, device, 16-byte aligned; scalar parameters are device values of
 * `dtype`, their gradients device fp32; reductions in a fixed order.
 *   Residual mixing before each block: y = lambdas[0] x + lambdas[1] x0
 *   (x0 the embedding output; n = N D elements, a multiple of 8).  Backout
 *   of a mid-layer residual x_mid after the last block is the same call
 *   with lambdas = (1, -backout_lambda) and x0 = x_mid.  Backward: dx =
 *   lambdas[0] dy (dx may be null; may alias dy), dx0 = (or +=, with
 *   accumulate) lambdas[1] dy, dlambdas[0] = sum dy x, dlambdas[1] = sum dy
 *   x0.  scratch: gpt_k_resid_mix_bwd_scratch_bytes().
 *   Smear after the embedding, rows of T tokens: y_t = x_t + g_t x_(t-1),
 *   g_t = lambda sigmoid(w . x_t[0:24]) (w: 24 values), g_t = 0 at each
 *   row's first position; gate[N] (fp32) keeps g for the backward.
 *   Backward: dx (not aliasing dy or x), dw_dlambda[0:24] = dw,
 *   dw_dlambda[24] = dlambda.  scratch: gpt_k_smear_bwd_scratch_bytes().
 *   D a multiple of 8 and >= 24. */
int gpt_k_resid_mix_fwd(const void* x, const void* x0, void* y, int64_t n,
                        const void* lambdas, int32_t dtype, hipStream_t s);
size_t gpt_k_resid_mix_bwd_scratch_bytes(void);
int gpt_k_resid_mix_bwd(const void* dy, const void* x, const void* x0,
                        void* dx, void* dx0, int32_t accumulate, int64_t n,
                        const void* lambdas, float* dlambdas, void* scratch,
                        size_t scratch_bytes, int32_t dtype, hipStream_t s);
int gpt_k_smear_fwd(const void* x, int32_t B, int32_t T, int32_t D,
                    const void* w, const void* lambda, void* y, float* gate,
                    int32_t dtype, hipStream_t s);
size_t gpt_k_smear_bwd_scratch_bytes(void);
int gpt_k_smear_bwd(const void* dy, const void* x, int32_t B, int32_t T,
                    int32_t D, const void* w, const void* lambda,
                    const float* gate, void* dx, float* dw_dlambda,
                    void* scratch, size_t scratch_bytes, int32_t dtype,
                    hipStream_t s);

/* cos/sin table, float2 [T, hd/2]: (cos, sin) of t * base^(-2j/hd),
 * evaluated in double precision. */
int gpt_k_rope_table(float* cs, int32_t T, int32_t hd, float base,
                     hipStream_t s);

/* In place on qkv [B*T, (H+2Hkv) hd]: rotate every q and k head, then RMS-
 * normalise it over hd; rq [B*T, H] and rk [B*T, Hkv] receive 1/rms. */
int gpt_k_rope_qknorm_fwd(void* qkv, float* rq, float* rk, const float* cs,
                          int32_t B, int32_t T, int32_t H, int32_t Hkv,
                          int32_t hd, float eps, int32_t dtype, hipStream_t s);

/* In place on the q and k parts of dqkv: norm backward (using the saved
 * normalised q/k of qkv and rq/rk), then the inverse rotation. */
int gpt_k_rope_qknorm_bwd(void* dqkv, const void* qkv, const float* rq,
                          const float* rk, const float* cs, int32_t B,
                          int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                          int32_t dtype, hipStream_t s);

/* Attention over qkv [B*T, (H+2Hkv) hd] -> o [B*T, H hd], lse [B, H, T];
 * causal, window `window` (keys i-window..i), query head h reads KV head
 * h / (H / Hkv); scale 1/sqrt(hd).  score_bound: 0, or a bound the caller
 * guarantees on every |q . k| / sqrt(hd) (rows after QK-norm: a little over
 * sqrt(hd)); with a bound the bf16 hd-128 kernel uses one fixed softmax
 * offset instead of a running maximum (scores above the bound by more than
 * ~80 would overflow).  Must lie in [0, 64), else GPT_ERR_INVALID_ARG. */
int gpt_k_attn_fwd(const void* qkv, void* o, float* lse, int32_t B,
                   int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                   int32_t window, int32_t dtype, float score_bound,
                   hipStream_t s);

/* Gradients of gpt_k_attn_fwd: dqkv (same layout as qkv) from do [B*T, H hd].
 * scratch: device, >= gpt_k_attn_bwd_scratch_bytes(B, T, H, hd) bytes. */
size_t gpt_k_attn_bwd_scratch_bytes(int32_t B, int32_t T, int32_t H,
                                    int32_t hd);
int gpt_k_attn_bwd(const void* qkv, const void* o, const float* lse,
                   const void* dout, void* dqkv, void* scratch, int32_t B,
                   int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                   int32_t window, int32_t dtype, hipStream_t s);

/* Attention of new tokens over a KV cache (generation: the nanochat
 * walkthrough, section "6. inference engine", prefilled caches read by
 * flash_attn_with_kvcache), bf16, head_dim 128.
 *   q [B, Tq, H, 128]: the Tq newest tokens of each sequence.
 *   k_cache, v_cache [B, Tmax, Hkv, 128]: sequence b holds positions
 *     0 .. L_b - 1, the new tokens' own keys and values included at
 *     L_b - Tq .. L_b - 1; rows at or past L_b are never read.
 *   cache_lens [B] int32 on the device: L_b, clamped to [0, Tmax].
 *   Query t of sequence b sits at position p = L_b - Tq + t and sees key j
 *   iff 0 <= p - j <= window; query head h reads KV head h / (H / Hkv);
 *   scale 1/sqrt(128).
 *   o [B, Tq, H, 128] bf16, lse [B, H, Tq] fp32 (natural log; a query with
 *   no visible key gets o = 0, lse = -inf).
 *   score_bound: as for gpt_k_attn_fwd, [0, 64).
 *   scratch: device, at least gpt_k_attn_decode_scratch_bytes(B, Tq, H, Hkv,
 *   Tmax, window) bytes (0 means none is needed), 16-byte aligned: arrival
 *   counters, then per-chunk partial results.  Zero-fill it once before its
 *   first use; every call leaves the counters at zero again, so the same
 *   buffer serves later calls without clearing.  Calls sharing a scratch
 *   buffer must not run concurrently.  Needs H % Hkv == 0, H / Hkv * Tq <= 1024, (Tmax + 64)
 *   * Hkv <= 2^24, B <= 65535 and Hkv * ceil(H / Hkv * Tq / 16) <= 65535.
 *   GPT_ERR_UNSUPPORTED_CONFIG for another dtype or head_dim, else
 *   GPT_ERR_INVALID_ARG / GPT_ERR_MISALIGNED / GPT_ERR_WORKSPACE_TOO_SMALL.
 *   Deterministic: fixed reduction order for given sizes. */
size_t gpt_k_attn_decode_scratch_bytes(int32_t B, int32_t Tq, int32_t H,
                                       int32_t Hkv, int32_t Tmax,
                                       int32_t window);
int gpt_k_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_lens, void* o, float* lse,
                      int32_t B, int32_t Tq, int32_t Tmax, int32_t H,
                      int32_t Hkv, int32_t hd, int32_t window,
                      float score_bound, void* scratch, size_t scratch_bytes,
                      int32_t dtype, hipStream_t s);

/* gpt_k_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without the scratch buffer.
 * Its scratch is a library-owned device array of
 * gpt_k_attn_decode_noalloc_max_scratch() bytes (8 MiB) per GPU, held
 * until the process ends.  Every size gpt_k_attn_decode accepts needs at
 * most 4,244,224 bytes of scratch, so all of them fit; a size whose
 * gpt_k_attn_decode_scratch_bytes() exceeded the array would return
 * GPT_ERR_INVALID_ARG before anything is enqueued.  The
 * call allocates nothing: it clears the array's counters with a kernel on
 * `s` (no memset node) and runs the decode kernel on it.  All calls on one
 * GPU share the array, so calls that overlap on one GPU (other streams, or
 * other threads) race; serialise them. */
size_t gpt_k_attn_decode_noalloc_max_scratch(void);
int gpt_k_attn_decode_noalloc(const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* cache_lens,
                              void* o, float* lse, int32_t B, int32_t Tq,
                              int32_t Tmax, int32_t H, int32_t Hkv, int32_t hd,
                              int32_t window, float score_bound, int32_t dtype,
                              hipStream_t s);

/* Token embedding (a1).  tokens [B, T+1] int32 (inputs are the first T of
 * each row), wte [V, D] dtype -> x [B*T, D] dtype: x[b*T + t] =
 * wte[tokens[b][t]] (bitwise copies of the rows). */
int gpt_k_embed_fwd(const int32_t* tokens, int32_t B, int32_t T,
                    const void* wte, int32_t V, int32_t D, void* x,
                    int32_t dtype, hipStream_t s);
/* Its gradient: dwte [V, D] fp32 (=, or += with accumulate = 1) the sum of
 * dx [B*T, D] (dtype) over the positions holding each id.  With scratch of
 * at least gpt_k_embed_bwd_scratch_bytes bytes (and D % 4 == 0, D <= 2048)
 * the ids are sorted once and every row summed in a fixed order
 * (deterministic); otherwise fp32 atomics. */
size_t gpt_k_embed_bwd_scratch_bytes(int32_t B, int32_t T, int32_t V,
                                     int32_t D);
int gpt_k_embed_bwd(const int32_t* tokens, int32_t B, int32_t T,
                    const void* dx, int32_t V, int32_t D, float* dwte,
                    int32_t accumulate, void* scratch, size_t scratch_bytes,
                    int32_t dtype, hipStream_t s);

/* Value embedding (a4), [nanochat] value-embedding snippet.  For every token
 * n (input id e = tokens[b][t]) and KV head kv: g[n, kv] = 3 sigmoid(
 * h[n, :C] . wg[kv, :]) (fp32 out, [B*T, Hkv]), and in place
 * qkv[n, voff + kv*hd + d] += g[n, kv] * E[e, kv*hd + d], rounded once.
 * h [B*T, D], wg [Hkv, C], E [V, Hkv*hd], qkv [B*T, ldqkv]; all dtype. */
int gpt_k_ve_fwd(const int32_t* tokens, int32_t B, int32_t T, const void* h,
                 int32_t D, const void* wg, int32_t C, const void* E,
                 void* qkv, int32_t ldqkv, int32_t voff, float* g,
                 int32_t Hkv, int32_t hd, int32_t dtype, hipStream_t s);
/* Its gradients from dv = dqkv[:, voff : voff + Hkv*hd]: vez [B*T, Hkv]
 * fp32 = (sum_d dv e) g (1 - g/3) (the gate pre-activation's gradient; its
 * share of dh[:, :C] is vez wg), dE [V, Hkv*hd] fp32 (=, or +=) the sum of
 * g dv over the positions holding each id, dwg [Hkv, C] fp32 (=, or +=)
 * vez^T h[:, :C].  scratch: at least gpt_k_ve_bwd_scratch_bytes bytes (the
 * sorted, deterministic table sum when the widths allow, else atomics). */
size_t gpt_k_ve_bwd_scratch_bytes(int32_t B, int32_t T, int32_t V, int32_t Hkv,
                                  int32_t hd, int32_t C);
int gpt_k_ve_bwd(const int32_t* tokens, int32_t B, int32_t T,
                 const void* dqkv, int32_t ldqkv, int32_t voff, const void* E,
                 const float* g, const void* h, int32_t D, int32_t C, int32_t V,
                 int32_t Hkv, int32_t hd, float* vez, float* dE, float* dwg,
                 int32_t accumulate, void* scratch, size_t scratch_bytes,
                 int32_t dtype, hipStream_t s);

/* Fused lm_head + softmax cross-entropy (bf16): logits = h [rows, D] times
 * w [V, D]^T are formed in fp32 inside the product and never stored; per
 * row and 256-column tile the product keeps the max and sum of exp(logit -
 * max) and writes exp(logit - max) as bf16 into dz, which a second pass
 * rescales in place (the same steps as the training step's loss).
 *   tgt[rows]: target ids in [0, V).  ell[row] = lse - logit[tgt[row]],
 *   lse[row] (fp32).  dz (may be null): [rows, V] bf16, receives
 *   (softmax - onehot) * grad_scale.  scratch: device, at least
 *   gpt_k_lm_ce_scratch_bytes(rows, V) bytes (per-tile statistics and target
 *   logits).  Needs V a multiple of 256, D a multiple of 64, h and w
 *   16-byte aligned (else GPT_ERR_INVALID_ARG / GPT_ERR_MISALIGNED). */
size_t gpt_k_lm_ce_scratch_bytes(int64_t rows, int32_t V);
int gpt_k_lm_ce(const void* h, const void* w, const int32_t* tgt, int64_t rows,
                int32_t D, int32_t V, float* ell, float* lse, void* dz,
                float grad_scale, void* scratch, hipStream_t s);

/* Softmax cross-entropy on fp32 logits z [rows, V] with targets tgt[rows]:
 * ell[row] = lse - z[tgt], lse[row]; if dz is non-null it receives
 * (softmax - onehot) * grad_scale in `dtype` [rows, V]. */
int gpt_k_ce(const float* z, const int32_t* tgt, int64_t rows, int32_t V,
             float* ell, float* lse, void* dz, float grad_scale,
             int32_t dtype, hipStream_t s);

/* ------------------------------------------------- launch recording */
/*
 * Per-launch timing of the library's own kernels, for measurement without a
 * profiler.  Between gpt_prof_start and gpt_prof_stop every kernel the
 * library enqueues (from any entry point above) is launched with
 * hipExtLaunchKernel and a start / stop HIP event pair that the runtime
 * ties to that kernel's dispatch on its stream, and its algorithmic work is
 * kept beside them: matmul flops (2 M N K for a product; for attention,
 * 2 hd per visible (query, key) pair and per matrix product the kernel
 * forms) and compulsory HBM bytes (operands read once, results written
 * once), 0 where not stated.  Recording adds event traffic per launch, so
 * time steps with recording off and use it for the per-kernel split.
 * Not for concurrent use from several host threads; events are owned by the
 * library until gpt_prof_clear or the next gpt_prof_start.
 */
/* Allocates 2*capacity events (host call, not enqueued), drops earlier
 * records and turns recording on.  GPT_ERR_INVALID_ARG unless
 * 1 <= capacity <= 2^20; GPT_ERR_HIP if event creation fails. */
int gpt_prof_start(int32_t capacity);
/* Turns recording off.  Returns 1 if launches beyond `capacity` went
 * unrecorded, else 0. */
int gpt_prof_stop(void);
/* Number of launches recorded. */
int32_t gpt_prof_count(void);
/* Record i (0-based, launch order): kernel name as the HIP runtime reports
 * it, demangled, truncated to name_len - 1 characters (host buffer);
 * duration in ms (waits for the launch to finish); flops and bytes as
 * above.  Only after gpt_prof_stop; GPT_ERR_INVALID_ARG for a bad index or
 * null output. */
int gpt_prof_record(int32_t i, char* name, size_t name_len, float* ms,
                    double* flops, double* bytes);
/* Turns recording off and frees the events and records. */
void gpt_prof_clear(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT_STEP_H */
