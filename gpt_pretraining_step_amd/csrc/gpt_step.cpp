// Host side of the GPT-step library: config validation, parameter layout,
// workspace planning, the forward / backward / eval launch sequences and the
// C ABI declared in include/gpt_step.h.
#include "gpt_step.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

// A debugging build (-DGPT_DEBUG_CHECKS) checks token ids on every call.
#ifdef GPT_DEBUG_CHECKS
static constexpr bool kDebugChecks = true;
#else
static constexpr bool kDebugChecks = false;
#endif
static constexpr int kMaxSideDevices = 64;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return fail(GPT_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));     \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t pad256(size_t b) { return (b + 255) & ~(size_t)255; }

// ------------------------------------------------------------- the model
struct Model {
  int L, D, H, Hkv, hd, V, T, B, F, C, QKV;
  int ve_odd;
  float base, eps;
  gk::DType dt;
  int es;                     // element size of the storage dtype
  std::string pattern;
  int wS, wL;
  // model extras: residual mixing, smear, backout after block `bo` (-1 off);
  // slots of the extras vector
  int resid, smear, bo;
  int ex_n, ex_sw, ex_sl, ex_bo;
  bool check_tokens;          // count out-of-range ids before any gather
  bool one_stream;            // backward on the caller's stream only

  bool extras() const { return resid || smear || bo >= 0; }

  bool is_ve(int l) const { return ve_odd && (l % 2 == 1); }
  int window(int l) const {
    if (pattern.empty()) return T;
    char c = pattern[l % pattern.size()];
    return c == 'S' ? wS : wL;
  }
};

int validate(const gpt_config* c, Model* m) {
  if (!c) return fail(GPT_ERR_INVALID_ARG, "config is null");
  if (c->n_layer < 1 || c->d_model < 1 || c->n_head < 1 || c->n_kv_head < 1 ||
      c->vocab < 2 || c->seq_len < 1 || c->batch < 1 || c->mlp_mult < 1)
    return fail(GPT_ERR_INVALID_ARG, "sizes must be positive (vocab >= 2)");
  if (c->n_head % c->n_kv_head)
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "n_head (%d) must be a multiple of n_kv_head (%d)",
                c->n_head, c->n_kv_head);
  int hd = c->head_dim;
  if (!(hd == 4 || hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128))
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "head_dim %d not in {4,8,16,32,64,128}", hd);
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16)
    return fail(GPT_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (!(c->norm_eps > 0.f) || !(c->rope_base > 0.f))
    return fail(GPT_ERR_INVALID_ARG, "norm_eps and rope_base must be positive");
  size_t plen = strnlen(c->window_pattern, sizeof(c->window_pattern));
  if (plen == sizeof(c->window_pattern))
    return fail(GPT_ERR_INVALID_ARG, "window_pattern is not NUL-terminated");
  for (size_t i = 0; i < plen; ++i)
    if (c->window_pattern[i] != 'S' && c->window_pattern[i] != 'L')
      return fail(GPT_ERR_INVALID_ARG, "window_pattern may hold only 'S' and 'L'");
  if (plen && (c->window_short < 0 || c->window_long < 0))
    return fail(GPT_ERR_INVALID_ARG, "windows must be >= 0");
  if (c->ve_every_odd && c->n_layer > 1 &&
      (c->ve_gate_channels < 1 || c->ve_gate_channels > c->d_model))
    return fail(GPT_ERR_INVALID_ARG, "ve_gate_channels must be in [1, d_model]");
  int64_t N = (int64_t)c->batch * c->seq_len;
  int64_t qkv = (int64_t)(c->n_head + 2 * c->n_kv_head) * hd;
  if (N > (1LL << 30) || (int64_t)c->mlp_mult * c->d_model > (1 << 30) || qkv > (1 << 30))
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "sizes too large");
  if (c->n_kv_head > 64) return fail(GPT_ERR_UNSUPPORTED_CONFIG, "n_kv_head > 64");
  if ((c->resid_lambdas != 0 && c->resid_lambdas != 1) || (c->smear != 0 && c->smear != 1) ||
      (c->backout != 0 && c->backout != 1))
    return fail(GPT_ERR_INVALID_ARG, "resid_lambdas, smear and backout must be 0 or 1");
  if (c->check_tokens != 0 && c->check_tokens != 1)
    return fail(GPT_ERR_INVALID_ARG, "check_tokens must be 0 or 1");
  if (c->one_stream != 0 && c->one_stream != 1)
    return fail(GPT_ERR_INVALID_ARG, "one_stream must be 0 or 1");
  if (c->backout && (c->backout_layer < 0 || c->backout_layer >= c->n_layer))
    return fail(GPT_ERR_INVALID_ARG, "backout_layer %d not in [0, n_layer)", c->backout_layer);
  if ((c->resid_lambdas || c->smear || c->backout) && c->d_model % 8)
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "model extras need d_model a multiple of 8");
  if (c->smear && c->d_model < 24)
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "smear reads 24 channels: d_model >= 24");
  if (m) {
    m->L = c->n_layer; m->D = c->d_model; m->H = c->n_head; m->Hkv = c->n_kv_head;
    m->hd = hd; m->V = c->vocab; m->T = c->seq_len; m->B = c->batch;
    m->F = c->mlp_mult * c->d_model; m->C = c->ve_gate_channels;
    m->QKV = (int)qkv; m->ve_odd = c->ve_every_odd ? 1 : 0;
    m->base = c->rope_base; m->eps = c->norm_eps;
    m->dt = c->dtype == GPT_BF16 ? gk::BF16 : gk::F32;
    m->es = c->dtype == GPT_BF16 ? 2 : 4;
    m->pattern.assign(c->window_pattern, plen);
    m->wS = c->window_short; m->wL = c->window_long;
    m->resid = c->resid_lambdas; m->smear = c->smear;
    m->bo = c->backout ? c->backout_layer : -1;
    m->ex_sw = 2 * m->L;
    m->ex_sl = 2 * m->L + 24;
    m->ex_bo = 2 * m->L + 25;
    m->ex_n = 8 * ((2 * m->L + 26 + 7) / 8);
    m->check_tokens = c->check_tokens != 0 || kDebugChecks;
    m->one_stream = c->one_stream != 0;
  }
  return GPT_OK;
}

// element offsets of every tensor in the flat parameter buffer
struct ParamLayout {
  int64_t wte, wlm, extras, total;     // extras: -1 when no extra is on
  std::vector<int64_t> wqkv, wo, wfc, wproj, ve, wg;
};

ParamLayout param_layout(const Model& m) {
  ParamLayout p;
  int64_t off = 0;
  p.wte = off; off += (int64_t)m.V * m.D;
  for (int l = 0; l < m.L; ++l) {
    p.wqkv.push_back(off); off += (int64_t)m.QKV * m.D;
    p.wo.push_back(off);   off += (int64_t)m.D * m.H * m.hd;
    p.wfc.push_back(off);  off += (int64_t)m.F * m.D;
    p.wproj.push_back(off); off += (int64_t)m.D * m.F;
    if (m.is_ve(l)) {
      p.ve.push_back(off); off += (int64_t)m.V * m.Hkv * m.hd;
      p.wg.push_back(off); off += (int64_t)m.Hkv * m.C;
    } else {
      p.ve.push_back(-1);
      p.wg.push_back(-1);
    }
  }
  p.wlm = off; off += (int64_t)m.V * m.D;
  p.extras = -1;
  if (m.extras()) { p.extras = off; off += m.ex_n; }
  p.total = off;
  return p;
}

// ------------------------------------------------------- workspace plan
struct LayerBufs {
  size_t h, r, qkv, rq, rk, g, o, lse, h2, r2, a;
};

struct Plan {
  int64_t N, chunk;
  size_t cs, x, hf, rf, ell, lse_z, loss, flag, badtok, logits, dz, evacc;
  bool fused_ce;         // lm_head + cross-entropy fused (no fp32 logits)
  // train, fused: the lm_head's input gradient is taken from e directly and
  // e is rescaled in place into the softmax gradient in the backward;
  // otherwise the gradient is formed in place over e in the forward
  bool ce_bwd;
  size_t ce_stats, ce_zt;
  std::vector<LayerBufs> layers;     // train: one per layer; eval: one shared
  // model extras: smear input and gates, the blocks' start x0, the stream
  // before each block's mix (train, blocks >= 1), the kept backout stream;
  // backward: x0's gradient, the kept stream's, the smear input's, and the
  // scalar gradients' partials
  size_t xe, sgate, x0, xmid, dx0, dxmid, dxe, ex_scr;
  std::vector<size_t> xpre;
  // backward scratch
  size_t dx, dh, du, dout, dqkv, attn_scr, vez, vwg, sort, gemm_scr, gemm_scr_bytes, wtp;
  bool sorted_scatter;   // embedding-table gradients by the token sort (no atomics)
  size_t total;
};

Plan make_plan(const Model& m, int mode) {
  Plan p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += pad256(bytes); return o; };
  const int64_t N = (int64_t)m.B * m.T;
  p.N = N;
  const size_t es = m.es;
  p.chunk = N;
  const int64_t max_logit_bytes = 512LL << 20;
  if (N * (int64_t)m.V * 4 > max_logit_bytes) {
    int64_t c = max_logit_bytes / ((int64_t)m.V * 4);
    c = (c / 256) * 256;
    if (c < 256) c = 256;
    p.chunk = c < N ? c : N;
  }
  p.cs = take((size_t)m.T * (m.hd / 2) * 8);
  p.x = take(N * m.D * es);
  p.hf = take(N * m.D * es);
  p.rf = take(N * 4);
  p.ell = take(N * 4);
  p.lse_z = take(N * 4);
  p.loss = take(4);
  p.flag = take(4);
  p.badtok = take(4);
  p.evacc = take(3 * 8);
  p.fused_ce = m.dt == gk::BF16 && gk::lm_ce_fused_ok(N, m.V, m.D);
  p.logits = p.fused_ce ? 0 : take((size_t)p.chunk * m.V * 4);
  p.ce_stats = p.fused_ce ? take(gk::lm_ce_stats_bytes(N, m.V)) : 0;
  p.ce_zt = p.fused_ce ? take(N * 4) : 0;
  p.dz = mode == GPT_MODE_TRAIN ? take((size_t)N * m.V * es) : 0;
  p.ce_bwd = p.fused_ce && mode == GPT_MODE_TRAIN && gk::lm_ce_bwd_ok(N, m.V, m.D);
  const bool train = mode == GPT_MODE_TRAIN;
  const size_t xbytes = (size_t)N * m.D * es;
  p.xe = m.smear ? take(xbytes) : 0;
  p.sgate = m.smear ? take(N * 4) : 0;
  p.x0 = m.resid ? take(xbytes) : 0;
  p.xmid = m.bo >= 0 ? take(xbytes) : 0;
  p.xpre.assign(m.L, 0);
  if (m.resid && train)
    for (int l = 1; l < m.L; ++l) p.xpre[l] = take(xbytes);
  p.dx0 = m.resid && train ? take(xbytes) : 0;
  p.dxmid = m.bo >= 0 && train ? take(xbytes) : 0;
  p.dxe = m.smear && train ? take(xbytes) : 0;
  p.ex_scr = m.extras() && train ? take(std::max(gk::resid_mix_bwd_scratch_bytes(),
                                                 gk::smear_bwd_scratch_bytes()))
                                 : 0;
  const int nl = mode == GPT_MODE_TRAIN ? m.L : 1;
  for (int l = 0; l < nl; ++l) {
    LayerBufs b;
    b.h = take(N * m.D * es);
    b.r = take(N * 4);
    b.qkv = take(N * (size_t)m.QKV * es);
    b.rq = take(N * (size_t)m.H * 4);
    b.rk = take(N * (size_t)m.Hkv * 4);
    b.g = take(N * (size_t)m.Hkv * 4);
    b.o = take(N * (size_t)m.H * m.hd * es);
    b.lse = take(N * (size_t)m.H * 4);
    b.h2 = take(N * m.D * es);
    b.r2 = take(N * 4);
    b.a = take(N * (size_t)m.F * es);
    p.layers.push_back(b);
  }
  if (mode == GPT_MODE_TRAIN) {
    p.dx = take(N * m.D * es);
    p.dh = take(N * m.D * es);
    p.du = take(N * (size_t)m.F * es);
    p.dout = take(N * (size_t)m.H * m.hd * es);
    p.dqkv = take(N * (size_t)m.QKV * es);
    p.attn_scr = take(gk::attn_bwd_scratch_bytes(m.B, m.T, m.H, m.hd));
    p.vez = take(N * (size_t)m.Hkv * 4);
    p.vwg = take(gk::ve_wgrad_scratch_bytes(m.Hkv, m.C));
    const int maxW = std::max(m.D, m.Hkv * m.hd);
    p.sorted_scatter = m.D % 4 == 0 && maxW <= 2048 && (m.Hkv * m.hd) % 4 == 0 && m.QKV % 4 == 0;
    p.sort = p.sorted_scatter ? take(gk::tok_sort_bytes(N, m.V, maxW)) : 0;
    // split-K partials of the weight-gradient products (largest of them)
    size_t gs = 0;
    const int64_t HD = (int64_t)m.H * m.hd;
    const int64_t shapes[5][2] = {{m.V, m.D}, {m.D, m.F}, {m.F, m.D}, {m.D, HD}, {m.QKV, m.D}};
    if (m.dt == gk::BF16)
      for (auto& sh : shapes) gs = std::max(gs, gk::gemm_scratch_bytes(sh[0], sh[1], N));
    p.gemm_scr_bytes = gs;
    p.gemm_scr = take(gs);
    // the transposed copy of W_proj for the MLP backward (its own buffer:
    // the weight-gradient products that use the split-K scratch may run at
    // the same time)
    p.wtp = m.dt == gk::BF16 ? take((size_t)m.F * m.D * 2) : 0;
  } else {
    p.dx = p.dh = p.du = p.dout = p.dqkv = p.attn_scr = p.vez = p.vwg = p.sort = p.gemm_scr = 0;
    p.wtp = 0;
    p.sorted_scatter = false;
    p.gemm_scr_bytes = 0;
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

const void* elem(const void* base, int64_t idx, int es) {
  return (const char*)base + idx * es;
}

// ------------------------------------------------------ launch sequences
// Forward over one batch of `rows` rows (rows <= m.B).  In TRAIN mode every
// layer's activations stay in ws for the backward; in EVAL mode one set of
// layer buffers is reused and no softmax gradient is formed.
int run_forward(const Model& m0, const Plan& p, const ParamLayout& pl, const void* params,
                const int32_t* tokens, int rows, void* ws, int mode, float* loss_dev,
                hipStream_t s) {
  Model m = m0;
  m.B = rows;
  const int64_t N = (int64_t)rows * m.T;
  const int es = m.es;
  const gk::DType dt = m.dt;
  void* x = at<void>(ws, p.x);            // the current block's stream
  void* const xfinal = x;                  // the last block's stream
  float* cs = at<float>(ws, p.cs);
  HIP_TRY(gk::rope_table(cs, m.T, m.hd, m.base, s));
  // with the extras the embedding feeds smear, whose output is x0 (or the
  // stream); mixing starts every block from the stream and x0
  void* xe = m.smear ? at<void>(ws, p.xe) : nullptr;
  void* x0 = m.resid ? at<void>(ws, p.x0) : nullptr;
  void* xmid = m.bo >= 0 ? at<void>(ws, p.xmid) : nullptr;
  const size_t xbytes = (size_t)N * m.D * es;
  HIP_TRY(gk::embed_fwd(tokens, rows, m.T, elem(params, pl.wte, es), xe ? xe : (x0 ? x0 : x),
                        m.D, dt, s));
  if (m.smear)
    HIP_TRY(gk::smear_fwd(xe, N, m.T, m.D, elem(params, pl.extras + m.ex_sw, es),
                          elem(params, pl.extras + m.ex_sl, es), x0 ? x0 : x,
                          at<float>(ws, p.sgate), dt, s));
  for (int l = 0; l < m.L; ++l) {
    const LayerBufs& b = p.layers[mode == GPT_MODE_TRAIN ? l : 0];
    void* h = at<void>(ws, b.h);
    void* qkv = at<void>(ws, b.qkv);
    void* o = at<void>(ws, b.o);
    void* h2 = at<void>(ws, b.h2);
    void* a = at<void>(ws, b.a);
    if (m.resid) {
      // stream = lr_l stream + l0_l x0 ahead of the block's norm (one pass
      // where the kernel allows).  In training each block has its own
      // stream buffer, so the stream before the mix (x0 for block 0) stays
      // for the backward: block l writes block l+1's pre-mix buffer (the
      // last block writes x); otherwise the mix works in place.
      const void* xin = l == 0 ? x0 : x;
      void* xo = mode == GPT_MODE_TRAIN && l < m.L - 1 ? at<void>(ws, p.xpre[l + 1]) : xfinal;
      const void* lam = elem(params, pl.extras + 2 * l, es);
      if (gk::rmsnorm_fwd_mix_ok(m.D, dt)) {
        HIP_TRY(gk::rmsnorm_fwd_mix(xin, x0, lam, xo, h, at<float>(ws, b.r), N, m.D, m.eps, dt,
                                    s));
      } else {
        HIP_TRY(gk::resid_mix_fwd(xin, x0, xo, N * m.D, lam, dt, s));
        HIP_TRY(gk::rmsnorm_fwd(xo, h, at<float>(ws, b.r), N, m.D, m.eps, dt, s));
      }
      x = xo;
    } else {
      HIP_TRY(gk::rmsnorm_fwd(x, h, at<float>(ws, b.r), N, m.D, m.eps, dt, s));
    }
    // RoPE then QK-norm touch only q and k, the value embedding only v: with
    // head_dim 128 the rotation and norm run in the QKV product's epilogue
    const bool qk_fused =
        dt == gk::BF16 && gk::qkv_rope_fused_ok(N, m.D, m.H, m.Hkv, m.hd) &&
        (!m.is_ve(l) || ((uintptr_t)elem(params, pl.ve[l], es) & 7) == 0);
    gk::GemmDesc g{gk::OP_NT, N, m.QKV, m.D, h, m.D, elem(params, pl.wqkv[l], es), m.D,
                   qkv, m.QKV, gk::E_STORE, nullptr};
    if (qk_fused) {
      // a value-embedding layer's v += g E[token] joins the same epilogue
      gk::VeArgs ve{tokens, m.is_ve(l) ? elem(params, pl.wg[l], es) : nullptr, m.C,
                    m.is_ve(l) ? elem(params, pl.ve[l], es) : nullptr, at<float>(ws, b.g)};
      HIP_TRY(gk::qkv_gemm_rope_norm(h, N, m.D, elem(params, pl.wqkv[l], es), m.H, m.Hkv, qkv,
                                     cs, at<float>(ws, b.rq), at<float>(ws, b.rk), m.T, m.eps,
                                     m.is_ve(l) ? &ve : nullptr, s));
    } else {
      HIP_TRY(gk::gemm(g, dt, s));
    }
    if (m.is_ve(l) && !qk_fused)
      HIP_TRY(gk::ve_fwd(tokens, rows, m.T, h, m.D, elem(params, pl.wg[l], es), m.C,
                         elem(params, pl.ve[l], es), qkv, m.QKV, (m.H + m.Hkv) * m.hd,
                         at<float>(ws, b.g), m.Hkv, m.hd, dt, s));
    if (!qk_fused)
      HIP_TRY(gk::rope_qknorm_fwd(qkv, at<float>(ws, b.rq), at<float>(ws, b.rk), cs, rows, m.T,
                                  m.H, m.Hkv, m.hd, m.eps, dt, s));
    // q and k rows are RMS-normalised (norm <= sqrt(hd), times 1 + 2^-8 per
    // factor after bf16 rounding), so |q . k| / sqrt(hd) <= 1.01 sqrt(hd)
    HIP_TRY(gk::attn_fwd(qkv, o, at<float>(ws, b.lse), rows, m.T, m.H, m.Hkv, m.hd, m.window(l),
                         dt, s, 1.01f * sqrtf((float)m.hd)));
    g = gk::GemmDesc{gk::OP_NT, N, m.D, (int64_t)m.H * m.hd, o, (int64_t)m.H * m.hd,
                     elem(params, pl.wo[l], es), (int64_t)m.H * m.hd, x, m.D, gk::E_RESADD,
                     nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    HIP_TRY(gk::rmsnorm_fwd(x, h2, at<float>(ws, b.r2), N, m.D, m.eps, dt, s));
    // only a = relu(u)^2 is kept (u rounded first); the backward takes
    // relu(u) as sqrt(a)
    g = gk::GemmDesc{gk::OP_NT, N, m.F, m.D, h2, m.D, elem(params, pl.wfc[l], es), m.D, a, m.F,
                     gk::E_RELU2, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    g = gk::GemmDesc{gk::OP_NT, N, m.D, m.F, a, m.F, elem(params, pl.wproj[l], es), m.F, x, m.D,
                     gk::E_RESADD, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    if (l == m.bo) HIP_TRY(hipMemcpyAsync(xmid, x, xbytes, hipMemcpyDeviceToDevice, s));
  }
  if (m.bo >= 0)
    HIP_TRY(gk::resid_mix_fwd(x, xmid, x, N * m.D, elem(params, pl.extras + m.ex_bo, es), dt, s,
                              gk::MIX_BACKOUT));
  void* hf = at<void>(ws, p.hf);
  HIP_TRY(gk::rmsnorm_fwd(x, hf, at<float>(ws, p.rf), N, m.D, m.eps, dt, s));
  float* logits = at<float>(ws, p.logits);
  const float inv_n = 1.0f / (float)N;
  if (p.fused_ce) {
    // TRAIN keeps e = exp(logit - tile max) for the backward (rescaled in
    // place into the softmax gradient here only when the backward cannot
    // take e as it is); EVAL keeps only the per-tile statistics
    void* e = mode == GPT_MODE_TRAIN ? at<void>(ws, p.dz) : nullptr;
    float* stats = at<float>(ws, p.ce_stats);
    float* zt = at<float>(ws, p.ce_zt);
    HIP_TRY(gk::lm_ce_gemm(hf, N, m.D, elem(params, pl.wlm, es), m.V, e, stats, zt, tokens, m.T,
                           0, s));
    HIP_TRY(gk::ce_fix(stats, zt, N, m.V, tokens, m.T, 0, at<float>(ws, p.ell),
                       at<float>(ws, p.lse_z), e, p.ce_bwd ? nullptr : e, inv_n, s));
  } else {
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t nr = N - r0 < p.chunk ? N - r0 : p.chunk;
    gk::GemmDesc g{gk::OP_NT, nr, m.V, m.D, elem(hf, r0 * m.D, es), m.D,
                   elem(params, pl.wlm, es), m.D, logits, m.V, gk::E_F32, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    // targets of rows r0.. : the ce kernel maps row -> token position itself
    void* dz = mode == GPT_MODE_TRAIN ? (void*)((char*)ws + p.dz + (size_t)r0 * m.V * es) : nullptr;
    HIP_TRY(gk::ce_rows(logits, nr, m.V, tokens, m.T, 0, at<float>(ws, p.ell) + r0,
                        at<float>(ws, p.lse_z) + r0, dz, inv_n, dt, s, r0));
  }
  }
  if (mode == GPT_MODE_TRAIN)
    HIP_TRY(gk::loss_reduce(at<float>(ws, p.ell), N, at<float>(ws, p.loss), loss_dev,
                            at<int>(ws, p.flag), s));
  return GPT_OK;
}

// The backward's second stream.  The weight-gradient products and the
// embedding-table and gate gradients are off the backward's critical path
// (nothing later reads them): they run on a library-owned stream, forked
// from the caller's stream where their inputs are ready and joined back
// before those inputs are overwritten and before the call returns, so they
// fill the caller stream's memory-bound kernels and kernel tails.  One
// stream and set of events per (host thread, device), created on first use
// and kept; default priority.  Results are bit for bit those of one stream
// (every kernel and its inputs are unchanged; only the overlap differs).
enum { EV_START, EV_DX1, EV_DX1_FREE, EV_DU, EV_DU_FREE, EV_DX2, EV_DX2_FREE, EV_QKV,
       EV_QKV_FREE, EV_END, EV_ATT_FORK, EV_ATT_JOIN, EV_ATT_JOIN4, EV_OPT_FORK, EV_OPT_J1,
       EV_OPT_J2, EV_OPT_J3, EV_COUNT };
struct SideStream {
  hipStream_t s = nullptr;
  hipStream_t s3 = nullptr;     // the attention backward's dQ pass
  hipStream_t s4 = nullptr;     // and its dV pass
  hipEvent_t ev[EV_COUNT] = {};
  bool ready = false, failed = false;
};
thread_local SideStream t_side[kMaxSideDevices];

// the side stream of the current device, or null (one stream then)
// split-K cap beside the main stream for weight-gradient products of fewer
// than 16 output tiles (W_o at d12: 9 tiles), whose partials are small:
// d12 step 33.84-33.90 ms against 33.94-34.02 with the common cap of 4
// (8: 33.93-33.97, 16: 33.92-33.95; one box)
static constexpr size_t kSmallSplitCap = 12;

SideStream* side_stream() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& ss = t_side[dev];
  if (ss.ready) return &ss;
  if (ss.failed) return nullptr;
  bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&ss.s3, hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&ss.s4, hipStreamNonBlocking) == hipSuccess;
  for (int i = 0; ok && i < EV_COUNT; ++i)
    ok = hipEventCreateWithFlags(&ss.ev[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    ss.failed = true;
    return nullptr;
  }
  ss.ready = true;
  return &ss;
}

int run_backward(const Model& m, const Plan& p, const ParamLayout& pl, const void* params,
                 const int32_t* tokens, void* ws, float* grads, int accumulate, hipStream_t s) {
  const int64_t N = p.N;
  const int es = m.es;
  const gk::DType dt = m.dt;
  const gk::Epi wepi = accumulate ? gk::E_F32_ACC : gk::E_F32;
  void* gscr = at<void>(ws, p.gemm_scr);
  const size_t gscr_bytes = p.gemm_scr_bytes;
  void* dx = at<void>(ws, p.dx);
  void* dh = at<void>(ws, p.dh);
  void* du = at<void>(ws, p.du);
  void* dout = at<void>(ws, p.dout);
  void* dqkv = at<void>(ws, p.dqkv);
  float* vez = at<float>(ws, p.vez);
  const float* cs = at<float>(ws, p.cs);
  const void* dz = at<void>(ws, p.dz);
  const void* hf = at<void>(ws, p.hf);
  // w: the stream of the off-path gradient work (the caller's stream when
  // the model is small or the side stream is unavailable)
  SideStream* sd = m.dt == gk::BF16 && N >= 4096 && !m.one_stream ? side_stream() : nullptr;
  const hipStream_t w = sd ? sd->s : s;
  // split-K scratch of a weight-gradient product [M_, N_].  Beside the main
  // stream these products need not fill the chip alone, and every split adds
  // partial-tile traffic: at most 4 splits there (d12 step: 33.56 ms against
  // 33.75 ms with the standalone plan's 7-28; 2 splits 38.1, 3 33.8, 5 33.6,
  // 6 33.9 ms, one box)
  auto wsb = [&](int64_t M_, int64_t N_) {
    const int64_t tiles = ((M_ + 255) / 256) * ((N_ + 255) / 256);
    const size_t cap = tiles < 16 ? kSmallSplitCap : 4;
    return sd ? std::min(gscr_bytes, cap * M_ * N_ * 4) : gscr_bytes;
  };
  bool marked[EV_COUNT] = {};
  auto fork = [&](int e) -> hipError_t {       // w waits for s's work so far
    if (!sd) return hipSuccess;
    hipError_t r = hipEventRecord(sd->ev[e], s);
    return r == hipSuccess ? hipStreamWaitEvent(w, sd->ev[e], 0) : r;
  };
  auto mark = [&](int e) -> hipError_t {       // a point in w's work
    if (!sd) return hipSuccess;
    marked[e] = true;
    return hipEventRecord(sd->ev[e], w);
  };
  auto need = [&](int e) -> hipError_t {       // s waits for w's work up to mark(e)
    if (!sd || !marked[e]) return hipSuccess;
    return hipStreamWaitEvent(s, sd->ev[e], 0);
  };

  // embedding tables: the batch's token ids are sorted once and every table
  // row is summed in a fixed order (rows of absent ids cleared unless
  // accumulating); otherwise they are scatter-added with atomics into
  // cleared tables
  const int maxW = std::max(m.D, m.Hkv * m.hd);
  void* sortws = at<void>(ws, p.sort);
  bool sorted = p.sorted_scatter && pl.wte % 4 == 0;      // 16-byte row stores
  for (int l = 0; l < m.L; ++l)
    if (m.is_ve(l)) sorted = sorted && pl.ve[l] % 4 == 0;
  if (sorted) {
    HIP_TRY(gk::tok_sort(tokens, m.B, m.T, m.V, maxW, sortws, s));
  } else if (!accumulate) {
    HIP_TRY(gk::fill_zero(grads + pl.wte, (int64_t)m.V * m.D * 4, s));
    for (int l = 0; l < m.L; ++l)
      if (m.is_ve(l)) HIP_TRY(gk::fill_zero(grads + pl.ve[l], (int64_t)m.V * m.Hkv * m.hd * 4, s));
  }
  // the extras' scalar gradients are added up over their kernels
  float* gex = m.extras() ? grads + pl.extras : nullptr;
  void* exscr = at<void>(ws, p.ex_scr);
  if (gex && !accumulate) HIP_TRY(gk::zero_f32(gex, m.ex_n, s));
  void* x0 = m.resid ? at<void>(ws, p.x0) : nullptr;
  void* dx0 = m.resid ? at<void>(ws, p.dx0) : nullptr;
  void* dxmid = m.bo >= 0 ? at<void>(ws, p.dxmid) : nullptr;
  // w starts after the token sort, the table clears, the forward and (fused
  // cross-entropy) the lm_head input gradient
  // lm_head.  With ce_bwd, dz holds e = exp(logit - m_t): the input
  // gradient's product reads e itself, then e is rescaled in place into the
  // softmax gradient (same stream, so after that product has read it) for
  // the weight gradient, which w takes from there.  Measured against the
  // rescale on w beside the input-gradient product: the two contend for
  // the CUs and the step is 0.13 ms slower
  const float inv_n = 1.0f / (float)N;
  gk::GemmDesc g{};
  if (p.ce_bwd) {
    HIP_TRY(gk::lm_ce_bwd_gemm(dz, N, m.V, elem(params, pl.wlm, es), m.D, dh,
                               at<float>(ws, p.ce_stats), at<float>(ws, p.lse_z), tokens, m.T, 0,
                               inv_n, s));
    HIP_TRY(gk::ce_fix(at<float>(ws, p.ce_stats), nullptr, N, m.V, tokens, m.T, 0, nullptr,
                       at<float>(ws, p.lse_z), dz, const_cast<void*>(dz), inv_n, s));
    HIP_TRY(fork(EV_START));
    g = gk::GemmDesc{gk::OP_TN, m.V, m.D, N, dz, m.V, hf, m.D, grads + pl.wlm, m.D, wepi, nullptr};
    HIP_TRY(gk::gemm(g, dt, w));
  } else {
    HIP_TRY(fork(EV_START));
    g = gk::GemmDesc{gk::OP_TN, m.V, m.D, N, dz, m.V, hf, m.D, grads + pl.wlm, m.D, wepi, nullptr};
    HIP_TRY(gk::gemm(g, dt, w));
    g = gk::GemmDesc{gk::OP_NN, N, m.D, m.V, dz, m.V, elem(params, pl.wlm, es), m.D, dh, m.D,
                     gk::E_STORE, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
  }
  HIP_TRY(gk::rmsnorm_bwd(dh, hf, at<float>(ws, p.rf), nullptr, dx, N, m.D, nullptr, nullptr, 0,
                          0, dt, s));
  // backout x -= lambda_b x_kept: dx passes through, the kept stream's
  // gradient is -lambda_b dx
  if (m.bo >= 0)
    HIP_TRY(gk::resid_mix_bwd(dx, nullptr, at<void>(ws, p.xmid), nullptr, dxmid, 0, N * m.D,
                              elem(params, pl.extras + m.ex_bo, es), gex + m.ex_bo, exscr, dt, s,
                              gk::MIX_BACKOUT, 1));
  for (int l = m.L - 1; l >= 0; --l) {
    const LayerBufs& b = p.layers[l];
    if (l == m.bo) HIP_TRY(gk::resid_mix_fwd(dx, dxmid, dx, N * m.D, nullptr, dt, s, gk::MIX_ADD));
    const void* h = at<void>(ws, b.h);
    const void* qkv = at<void>(ws, b.qkv);
    const void* o = at<void>(ws, b.o);
    const void* h2 = at<void>(ws, b.h2);
    const void* a = at<void>(ws, b.a);
    const int64_t HD = (int64_t)m.H * m.hd;
    // MLP
    HIP_TRY(fork(EV_DX1));                      // dx (the block output's gradient) ready
    g = gk::GemmDesc{gk::OP_TN, m.D, m.F, N, dx, m.D, a, m.F, grads + pl.wproj[l], m.F, wepi,
                     nullptr, gscr, wsb(m.D, m.F)};
    HIP_TRY(gk::gemm(g, dt, w));
    HIP_TRY(mark(EV_DX1_FREE));
    HIP_TRY(need(EV_DU_FREE));                  // the previous block's dW_fc has read du
    if (dt == gk::BF16 && m.F % 8 == 0 && m.D % 8 == 0) {
      // du = (dx W_proj) * 2 sqrt(a) as an NT product against W_proj^T:
      // the K-contiguous operand reads run faster than the transposing ones
      void* wtp = at<void>(ws, p.wtp);
      HIP_TRY(gk::transpose_bf16(elem(params, pl.wproj[l], es), m.D, m.F, wtp, s));
      g = gk::GemmDesc{gk::OP_NT, N, m.F, m.D, dx, m.D, wtp, m.D, du, m.F, gk::E_DRELU2,
                       const_cast<void*>(a)};
    } else {
      g = gk::GemmDesc{gk::OP_NN, N, m.F, m.D, dx, m.D, elem(params, pl.wproj[l], es), m.F, du,
                       m.F, gk::E_DRELU2, const_cast<void*>(a)};
    }
    HIP_TRY(gk::gemm(g, dt, s));
    HIP_TRY(fork(EV_DU));
    g = gk::GemmDesc{gk::OP_TN, m.F, m.D, N, du, m.F, h2, m.D, grads + pl.wfc[l], m.D, wepi,
                     nullptr, gscr, wsb(m.F, m.D)};
    HIP_TRY(gk::gemm(g, dt, w));
    HIP_TRY(mark(EV_DU_FREE));
    g = gk::GemmDesc{gk::OP_NN, N, m.D, m.F, du, m.F, elem(params, pl.wfc[l], es), m.D, dh, m.D,
                     gk::E_STORE, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    HIP_TRY(need(EV_DX1_FREE));                 // dW_proj has read dx
    HIP_TRY(gk::rmsnorm_bwd(dh, h2, at<float>(ws, b.r2), dx, dx, N, m.D, nullptr, nullptr, 0, 0,
                            dt, s));
    // attention
    HIP_TRY(fork(EV_DX2));
    g = gk::GemmDesc{gk::OP_TN, m.D, HD, N, dx, m.D, o, HD, grads + pl.wo[l], HD, wepi, nullptr, gscr, wsb(m.D, HD)};
    HIP_TRY(gk::gemm(g, dt, w));
    HIP_TRY(mark(EV_DX2_FREE));
    g = gk::GemmDesc{gk::OP_NN, N, HD, m.D, dx, m.D, elem(params, pl.wo[l], es), HD, dout, HD,
                     gk::E_STORE, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    HIP_TRY(need(EV_QKV_FREE));                 // the previous block's users of dqkv, vez are done
    // attention backward; where the kernels can, they also apply the
    // backward of RoPE-then-QK-norm in their epilogues
    if (gk::attn_bwd_fuses_norm(m.T, m.H, m.Hkv, m.hd, dt)) {
      gk::Beside bes;
      if (sd)
        bes = gk::Beside{sd->s3, sd->ev[EV_ATT_FORK], sd->ev[EV_ATT_JOIN], sd->s4,
                         sd->ev[EV_ATT_JOIN4]};
      HIP_TRY(gk::attn_bwd(qkv, o, at<float>(ws, b.lse), dout, dqkv, at<void>(ws, p.attn_scr),
                           m.B, m.T, m.H, m.Hkv, m.hd, m.window(l), dt, s, at<float>(ws, b.rq),
                           at<float>(ws, b.rk), cs, bes));
    } else {
      HIP_TRY(gk::attn_bwd(qkv, o, at<float>(ws, b.lse), dout, dqkv, at<void>(ws, p.attn_scr),
                           m.B, m.T, m.H, m.Hkv, m.hd, m.window(l), dt, s));
      HIP_TRY(gk::rope_qknorm_bwd(dqkv, qkv, at<float>(ws, b.rq), at<float>(ws, b.rk), cs, m.B,
                                  m.T, m.H, m.Hkv, m.hd, dt, s));
    }
    const bool ve = m.is_ve(l);
    if (ve) {
      const int voff = (m.H + m.Hkv) * m.hd;
      if (sorted) {
        HIP_TRY(gk::ve_vez(tokens, m.B, m.T, dqkv, m.QKV, voff, elem(params, pl.ve[l], es),
                           at<float>(ws, b.g), vez, m.Hkv, m.hd, dt, s));
        HIP_TRY(fork(EV_QKV));
        HIP_TRY(gk::seg_scatter(sortws, N, m.V, maxW, elem(dqkv, voff, es), m.QKV,
                                m.Hkv * m.hd, at<float>(ws, b.g), m.Hkv, m.hd, grads + pl.ve[l],
                                accumulate, dt, w));
      } else {
        HIP_TRY(gk::ve_bwd(tokens, m.B, m.T, dqkv, m.QKV, voff, elem(params, pl.ve[l], es),
                           at<float>(ws, b.g), vez, grads + pl.ve[l], m.Hkv, m.hd, dt, s));
        HIP_TRY(fork(EV_QKV));
      }
      HIP_TRY(gk::ve_wgrad(vez, h, m.D, N, m.Hkv, m.C, grads + pl.wg[l], accumulate,
                           at<float>(ws, p.vwg), dt, w));
    } else {
      HIP_TRY(fork(EV_QKV));
    }
    g = gk::GemmDesc{gk::OP_TN, m.QKV, m.D, N, dqkv, m.QKV, h, m.D, grads + pl.wqkv[l], m.D,
                     wepi, nullptr, gscr, wsb(m.QKV, m.D)};
    HIP_TRY(gk::gemm(g, dt, w));
    HIP_TRY(mark(EV_QKV_FREE));
    g = gk::GemmDesc{gk::OP_NN, N, m.D, m.QKV, dqkv, m.QKV, elem(params, pl.wqkv[l], es), m.D,
                     dh, m.D, gk::E_STORE, nullptr};
    HIP_TRY(gk::gemm(g, dt, s));
    HIP_TRY(need(EV_DX2_FREE));                 // dW_o has read dx
    HIP_TRY(gk::rmsnorm_bwd(dh, h, at<float>(ws, b.r), dx, dx, N, m.D, ve ? vez : nullptr,
                            ve ? elem(params, pl.wg[l], es) : nullptr, m.Hkv, m.C, dt, s));
    // mix x = lr_l x_pre + l0_l x0: dx_pre = lr_l dx, x0's gradient gathers
    // l0_l dx over the blocks
    if (m.resid)
      HIP_TRY(gk::resid_mix_bwd(dx, l == 0 ? x0 : at<void>(ws, p.xpre[l]), x0, dx, dx0,
                                l < m.L - 1, N * m.D, elem(params, pl.extras + 2 * l, es),
                                gex + 2 * l, exscr, dt, s, gk::MIX_LAMBDAS, 1));
  }
  if (m.resid) HIP_TRY(gk::resid_mix_fwd(dx, dx0, dx, N * m.D, nullptr, dt, s, gk::MIX_ADD));
  void* demb = dx;
  if (m.smear) {
    demb = at<void>(ws, p.dxe);
    HIP_TRY(gk::smear_bwd(dx, at<void>(ws, p.xe), N, m.T, m.D,
                          elem(params, pl.extras + m.ex_sw, es),
                          elem(params, pl.extras + m.ex_sl, es), at<float>(ws, p.sgate), demb,
                          gex + m.ex_sw, exscr, dt, s, 1));
  }
  if (sorted)
    HIP_TRY(gk::seg_scatter(sortws, N, m.V, maxW, demb, m.D, m.D, nullptr, 1, m.D,
                            grads + pl.wte, accumulate, dt, s));
  else
    HIP_TRY(gk::embed_bwd(tokens, m.B, m.T, demb, m.D, grads + pl.wte, m.D, dt, s));
  // everything on w is done before the caller's stream moves on
  HIP_TRY(mark(EV_END));
  HIP_TRY(need(EV_END));
  return GPT_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* q : ps) {
    if (!q) return fail(GPT_ERR_INVALID_ARG, "a required pointer is null");
    if (!aligned16(q)) return fail(GPT_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
  }
  return GPT_OK;
}

// ------------------------------ decode attention without allocation
// The split-key scratch of gpt_k_attn_decode (arrival counters, then the
// chunks' partial records) in a fixed-size device array instead of a caller
// buffer, for callers that cannot allocate (graph capture, serving loops).
// Each GPU holds its own copy of the array; host code reaches it only
// through the device address looked up below, once per device.  The decode
// plan caps the records at 510 chunk records of 16 query slots x 130 floats
// (plus 1 KB of counters): 4,244,224 bytes, so every size the regular entry
// accepts fits.
constexpr size_t kDecodeScratchMax = (size_t)8 << 20;      // bytes per GPU
static __device__ __align__(256) unsigned char decode_scratch[kDecodeScratchMax];
constexpr int kMaxDevices = 64;
void* g_decode_scratch[kMaxDevices];
std::mutex g_decode_scratch_mu;

// The array's address on the current device (looked up with that device
// current, the first time it is asked for there).
int decode_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GPT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GPT_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_decode_scratch_mu);
  if (!g_decode_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch));
    if (e != hipSuccess || !p)
      return fail(GPT_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_decode_scratch[dev] = p;
  }
  *out = g_decode_scratch[dev];
  return GPT_OK;
}

}  // namespace

// =============================================================== C ABI
extern "C" {

int gpt_validate_config(const gpt_config* cfg) { return validate(cfg, nullptr); }

int64_t gpt_param_count(const gpt_config* cfg) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  return param_layout(m).total;
}

int64_t gpt_param_offset(const gpt_config* cfg, int which, int layer) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  ParamLayout p = param_layout(m);
  if (which == GPT_P_WTE) return p.wte;
  if (which == GPT_P_WLM) return p.wlm;
  if (which == GPT_P_EXTRAS) return p.extras;
  if (layer < 0 || layer >= m.L) return fail(GPT_ERR_INVALID_ARG, "layer out of range");
  switch (which) {
    case GPT_P_WQKV: return p.wqkv[layer];
    case GPT_P_WO: return p.wo[layer];
    case GPT_P_WFC: return p.wfc[layer];
    case GPT_P_WPROJ: return p.wproj[layer];
    case GPT_P_VE: return p.ve[layer];
    case GPT_P_WG: return p.wg[layer];
  }
  return fail(GPT_ERR_INVALID_ARG, "unknown tensor id %d", which);
}

size_t gpt_workspace_bytes(const gpt_config* cfg, int mode) {
  Model m;
  if (validate(cfg, &m)) return 0;
  if (mode != GPT_MODE_TRAIN && mode != GPT_MODE_EVAL) {
    fail(GPT_ERR_INVALID_ARG, "unknown workspace mode %d", mode);
    return 0;
  }
  return make_plan(m, mode).total;
}

int64_t gpt_ws_offset(const gpt_config* cfg, int which, int layer) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  Plan p = make_plan(m, GPT_MODE_TRAIN);
  switch (which) {
    case GPT_WS_ELL: return (int64_t)p.ell;
    case GPT_WS_LOSS: return (int64_t)p.loss;
    case GPT_WS_NONFINITE: return (int64_t)p.flag;
    case GPT_WS_X_HF: return (int64_t)p.hf;
    case GPT_WS_BAD_TOKENS: return (int64_t)p.badtok;
  }
  if (layer < 0 || layer >= m.L) return fail(GPT_ERR_INVALID_ARG, "layer out of range");
  const LayerBufs& b = p.layers[layer];
  switch (which) {
    case GPT_WS_X_H: return (int64_t)b.h;
    case GPT_WS_X_QKV: return (int64_t)b.qkv;
    case GPT_WS_X_O: return (int64_t)b.o;
    case GPT_WS_X_LSE: return (int64_t)b.lse;
    case GPT_WS_X_H2: return (int64_t)b.h2;
    case GPT_WS_X_A: return (int64_t)b.a;
  }
  return fail(GPT_ERR_INVALID_ARG, "unknown workspace item %d", which);
}

// With the token check on: count the ids outside [0, V) on the device,
// wait for the count, and refuse the call before any gather is enqueued.
static int check_token_ids(const Model& m, const Plan& p, const int32_t* tokens, int64_t n,
                           void* ws, hipStream_t stream) {
  if (!m.check_tokens) return GPT_OK;
  int* dcount = at<int>(ws, p.badtok);
  hipError_t e = gk::count_bad_ids(tokens, n, m.V, dcount, stream);
  int bad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, dcount, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GPT_ERR_HIP, "token check: %s", hipGetErrorString(e));
  if (bad) return fail(GPT_ERR_INVALID_ARG, "%d token ids outside [0, %d)", bad, m.V);
  return GPT_OK;
}

int gpt_step_fwd(const gpt_config* cfg, const void* params, const int32_t* tokens, void* ws,
                 size_t ws_bytes, float* loss_dev, hipStream_t stream) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  if ((st = check_ptrs({params, tokens, ws, loss_dev}))) return st;
  Plan p = make_plan(m, GPT_MODE_TRAIN);
  if (ws_bytes < p.total)
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if ((st = check_token_ids(m, p, tokens, (int64_t)m.B * (m.T + 1), ws, stream))) return st;
  return run_forward(m, p, param_layout(m), params, tokens, m.B, ws, GPT_MODE_TRAIN, loss_dev,
                     stream);
}

int gpt_step_bwd(const gpt_config* cfg, const void* params, const int32_t* tokens, void* ws,
                 size_t ws_bytes, float* grads, int accumulate, hipStream_t stream) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  if ((st = check_ptrs({params, tokens, ws, grads}))) return st;
  if (accumulate != 0 && accumulate != 1)
    return fail(GPT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  Plan p = make_plan(m, GPT_MODE_TRAIN);
  if (ws_bytes < p.total)
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if ((st = check_token_ids(m, p, tokens, (int64_t)m.B * (m.T + 1), ws, stream))) return st;
  return run_backward(m, p, param_layout(m), params, tokens, ws, grads, accumulate, stream);
}

int gpt_eval_bpb(const gpt_config* cfg, const void* params, const int32_t* tokens,
                 int64_t n_rows, const int32_t* token_bytes, void* ws, size_t ws_bytes,
                 double* out_dev, hipStream_t stream) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  if ((st = check_ptrs({params, tokens, token_bytes, ws, out_dev}))) return st;
  if (n_rows < 1) return fail(GPT_ERR_INVALID_ARG, "n_rows must be >= 1");
  Plan p = make_plan(m, GPT_MODE_EVAL);
  if (ws_bytes < p.total)
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, p.total);
  if ((st = check_token_ids(m, p, tokens, n_rows * (m.T + 1), ws, stream))) return st;
  ParamLayout pl = param_layout(m);
  double* acc = at<double>(ws, p.evacc);
  for (int64_t r0 = 0; r0 < n_rows; r0 += m.B) {
    int rows = (int)(n_rows - r0 < m.B ? n_rows - r0 : m.B);
    const int32_t* tk = tokens + r0 * (m.T + 1);
    st = run_forward(m, p, pl, params, tk, rows, ws, GPT_MODE_EVAL, nullptr, stream);
    if (st) return st;
    hipError_t e = gk::eval_accum(at<float>(ws, p.ell), tk, rows, m.T, token_bytes, acc, r0 == 0,
                                  stream);
    if (e != hipSuccess) return fail(GPT_ERR_HIP, "eval_accum: %s", hipGetErrorString(e));
  }
  hipError_t e = gk::eval_finish(acc, out_dev, stream);
  if (e != hipSuccess) return fail(GPT_ERR_HIP, "eval_finish: %s", hipGetErrorString(e));
  return GPT_OK;
}

// ------------------------------------------------------- optimizer step
namespace {
struct MuonGroup {
  const std::vector<int64_t>* offs;
  int64_t rows, cols;
};
std::vector<MuonGroup> muon_groups(const Model& m, const ParamLayout& pl) {
  return {{&pl.wqkv, m.QKV, m.D}, {&pl.wo, m.D, (int64_t)m.H * m.hd},
          {&pl.wfc, m.F, m.D}, {&pl.wproj, m.D, m.F}};
}
// the optimizer workspace of one Muon group (staging copy, orthogonalized
// update, orthogonalization / NorMuon scratch); the groups get disjoint
// regions so they can run side by side
size_t muon_group_ws(const Model& m, const MuonGroup& g) {
  const size_t n = (size_t)m.L * g.rows * g.cols;
  const size_t stage = (n * 4 + 255) / 256 * 256, xb = (n * 2 + 255) / 256 * 256;
  const size_t scr = std::max(gk::polar_express_ws_bytes(m.L, g.rows, g.cols),
                              gk::normuon_scratch_bytes(m.L, g.rows));
  return stage + xb + (scr + 255) / 256 * 256;
}

size_t optim_ws(const Model& m, const ParamLayout& pl) {
  size_t b = 0;
  for (const MuonGroup& g : muon_groups(m, pl)) b += muon_group_ws(m, g);
  return b;
}
}  // namespace

size_t gpt_optim_ws_bytes(const gpt_config* cfg) {
  Model m;
  if (validate(cfg, &m)) return 0;
  return optim_ws(m, param_layout(m));
}

int gpt_optim_step(const gpt_config* cfg, const gpt_optim_hparams* hp, int32_t step,
                   float* master, void* params, const float* grads, float* state1,
                   float* state2, void* ws, size_t ws_bytes, hipStream_t s) {
  Model m;
  int st = validate(cfg, &m);
  if (st) return st;
  if (!hp) return fail(GPT_ERR_INVALID_ARG, "hparams is null");
  if ((st = check_ptrs({master, grads, state1, state2, ws}))) return st;
  if (params && !aligned16(params)) return fail(GPT_ERR_MISALIGNED, "params misaligned");
  if (m.dt == gk::BF16 && !params)
    return fail(GPT_ERR_INVALID_ARG, "bf16 configs need the params copy to update");
  if (step < 1) return fail(GPT_ERR_INVALID_ARG, "step counts from 1");
  if (hp->ns_steps < 0 || hp->ns_steps > 16)
    return fail(GPT_ERR_INVALID_ARG, "ns_steps outside [0, 16]");
  if (hp->normuon && !(hp->normuon_beta2 >= 0.f && hp->normuon_beta2 < 1.f))
    return fail(GPT_ERR_INVALID_ARG, "normuon_beta2 outside [0, 1)");
  if (!(hp->muon_momentum >= 0.f && hp->muon_momentum < 1.f) ||
      !(hp->adam_beta1 >= 0.f && hp->adam_beta1 < 1.f) ||
      !(hp->adam_beta2 >= 0.f && hp->adam_beta2 < 1.f))
    return fail(GPT_ERR_INVALID_ARG, "momentum or betas outside [0, 1)");
  const ParamLayout pl = param_layout(m);
  const size_t need = optim_ws(m, pl);
  if (ws_bytes < need) return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "ws needs %zu bytes", need);
  // every tensor starts on a 16-byte boundary in both copies
  auto ok_off = [&](int64_t off) { return off < 0 || off % 8 == 0; };
  bool aligned = ok_off(pl.wte) && ok_off(pl.wlm) && ok_off(pl.extras);
  for (int l = 0; l < m.L; ++l)
    aligned = aligned && ok_off(pl.wqkv[l]) && ok_off(pl.wo[l]) && ok_off(pl.wfc[l]) &&
              ok_off(pl.wproj[l]) && ok_off(pl.ve[l]) && ok_off(pl.wg[l]);
  if (!aligned || m.D % 8 || m.F % 8 || m.QKV % 8 || (m.H * m.hd) % 8)
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "parameter tensors not 8-element aligned");
  const bool copy16 = m.dt == gk::BF16;
  auto p16 = [&](int64_t off) { return copy16 ? (void*)((char*)params + off * 2) : nullptr; };
  char* w = (char*)ws;
  // The Muon groups (one per weight shape) are independent: beside the
  // caller's stream they run on the library's side streams, forked from and
  // joined back into it with events, each in its own workspace region (the
  // small Newton-Schulz products of one group leave most CUs idle)
  SideStream* sd = m.dt == gk::BF16 && !m.one_stream ? side_stream() : nullptr;
  const std::vector<MuonGroup> groups = muon_groups(m, pl);
  hipStream_t gs[4] = {s, s, s, s};
  if (sd && groups.size() <= 4) {
    HIP_TRY(hipEventRecord(sd->ev[EV_OPT_FORK], s));
    const hipStream_t side[3] = {sd->s, sd->s3, sd->s4};
    for (size_t i = 1; i < groups.size(); ++i) {
      gs[i] = side[i - 1];
      HIP_TRY(hipStreamWaitEvent(gs[i], sd->ev[EV_OPT_FORK], 0));
    }
  }
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const MuonGroup& g = groups[gi];
    const hipStream_t s = gs[gi];
    const int64_t n = g.rows * g.cols;
    const size_t stage = ((size_t)m.L * n * 4 + 255) / 256 * 256;
    const size_t xb = ((size_t)m.L * n * 2 + 255) / 256 * 256;
    float* u = (float*)w;
    uint16_t* x = (uint16_t*)(w + stage);
    void* nsws = w + stage + xb;
    w += muon_group_ws(m, g);
    // momentum and update run over the group's L matrices in one launch each
    // (per matrix for deeper models than the offset table holds)
    const bool grouped = m.L <= gk::kMaxGroupLayers;
    gk::LayerOffsets offs{};
    for (int l = 0; grouped && l < m.L; ++l) offs.off[l] = (*g.offs)[l];
    if (grouped) {
      HIP_TRY(gk::muon_momentum_group(grads, state1, u, offs, m.L, n, hp->muon_momentum,
                                      hp->muon_nesterov ? 1 : 0, gk::F32, s));
    } else {
      for (int l = 0; l < m.L; ++l) {
        const int64_t off = (*g.offs)[l];
        HIP_TRY(gk::muon_momentum(grads + off, state1 + off, u + l * n, n, hp->muon_momentum,
                                  hp->muon_nesterov ? 1 : 0, gk::F32, s));
      }
    }
    HIP_TRY(gk::polar_express(u, m.L, g.rows, g.cols, gk::F32, hp->ns_coeffs, hp->ns_steps,
                              hp->ns_eps, x, nsws, s));
    const float lr = hp->muon_lr * std::sqrt(std::max(1.0f, (float)g.rows / (float)g.cols));
    if (hp->normuon) {
      // NorMuon: per-row second moments in state2 (the first `rows` floats
      // of each matrix's slot, unused by Muon otherwise); the statistics'
      // scratch reuses the orthogonalization's workspace, done by now
      if (grouped) {
        HIP_TRY(gk::normuon_update_group(master, x, state2, offs, m.L, g.rows, g.cols,
                                         hp->normuon_beta2, lr, hp->muon_wd,
                                         copy16 ? params : nullptr, nsws, s));
      } else {
        for (int l = 0; l < m.L; ++l) {
          gk::LayerOffsets one{};
          one.off[0] = (*g.offs)[l];
          HIP_TRY(gk::normuon_update_group(master, x + l * n, state2, one, 1, g.rows, g.cols,
                                           hp->normuon_beta2, lr, hp->muon_wd,
                                           copy16 ? params : nullptr, nsws, s));
        }
      }
    } else if (grouped) {
      HIP_TRY(gk::muon_update_group(master, x, offs, m.L, n, lr, hp->muon_wd,
                                    copy16 ? params : nullptr, s));
    } else {
      for (int l = 0; l < m.L; ++l) {
        const int64_t off = (*g.offs)[l];
        HIP_TRY(gk::muon_update(master + off, x + l * n, n, lr, hp->muon_wd, p16(off), s));
      }
    }
  }
  // AdamW (on the caller's stream, beside the side streams' groups):
  // embeddings and value-embedding tables, lm_head, gates, extras
  auto adam = [&](int64_t off, int64_t n, float lr) -> int {
    HIP_TRY(gk::adamw(master + off, grads + off, state1 + off, state2 + off, n, step, lr,
                      hp->adam_beta1, hp->adam_beta2, hp->adam_eps, hp->adam_wd, p16(off), s));
    return GPT_OK;
  };
  if ((st = adam(pl.wte, (int64_t)m.V * m.D, hp->adam_lr_embed))) return st;
  if ((st = adam(pl.wlm, (int64_t)m.V * m.D, hp->adam_lr_head))) return st;
  for (int l = 0; l < m.L; ++l) {
    if (pl.ve[l] < 0) continue;
    if ((st = adam(pl.ve[l], (int64_t)m.V * m.Hkv * m.hd, hp->adam_lr_embed))) return st;
    if ((st = adam(pl.wg[l], (int64_t)m.Hkv * m.C, hp->adam_lr_gate))) return st;
  }
  // the model extras' scalars and smear weights, with the gates
  if (pl.extras >= 0 && (st = adam(pl.extras, m.ex_n, hp->adam_lr_gate))) return st;
  // the caller's stream waits for the side streams' groups
  const int joins[3] = {EV_OPT_J1, EV_OPT_J2, EV_OPT_J3};
  for (size_t i = 1; i < groups.size(); ++i) {
    if (gs[i] == s) continue;
    HIP_TRY(hipEventRecord(sd->ev[joins[i - 1]], gs[i]));
    HIP_TRY(hipStreamWaitEvent(s, sd->ev[joins[i - 1]], 0));
  }
  return GPT_OK;
}

const char* gpt_status_string(int status) {
  switch (status) {
    case GPT_OK: return "ok";
    case GPT_ERR_INVALID_ARG: return "invalid argument";
    case GPT_ERR_UNSUPPORTED_CONFIG: return "unsupported config";
    case GPT_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GPT_ERR_MISALIGNED: return "misaligned pointer";
    case GPT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* gpt_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------- kernel entries
static int dtype_ok(int32_t dtype) {
  if (dtype != GPT_F32 && dtype != GPT_BF16) return fail(GPT_ERR_INVALID_ARG, "unknown dtype");
  return GPT_OK;
}
#define KERNEL_TRY(expr)                                                           \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) return fail(GPT_ERR_HIP, "%s", hipGetErrorString(e_));   \
  } while (0)

int gpt_k_rmsnorm_fwd(const void* x, void* y, float* r, int64_t rows, int32_t dim, float eps,
                      int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({x, y, r}))) return st;
  if (rows < 0 || dim < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::rmsnorm_fwd(x, y, r, rows, dim, eps, (gk::DType)dtype, s));
  return GPT_OK;
}

int gpt_k_rmsnorm_bwd(const void* dy, const void* y, const float* r, const void* dres, void* dx,
                      int64_t rows, int32_t dim, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({dy, y, r, dx}))) return st;
  if (dres && !aligned16(dres)) return fail(GPT_ERR_MISALIGNED, "dres misaligned");
  if (rows < 0 || dim < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::rmsnorm_bwd(dy, y, r, dres, dx, rows, dim, nullptr, nullptr, 0, 0,
                             (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_gemm_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return gk::gemm_scratch_bytes(M, N, K);
}

int gpt_k_gemm(int32_t op, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
               const void* B, int64_t ldb, void* C, int64_t ldc, int32_t epilogue, void* aux,
               void* scratch, size_t scratch_bytes, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({A, B, C}))) return st;
  if (op < GPT_GEMM_NT || op > GPT_GEMM_TN) return fail(GPT_ERR_INVALID_ARG, "unknown op");
  if (epilogue < GPT_EPI_STORE || epilogue > GPT_EPI_F32_ACC)
    return fail(GPT_ERR_INVALID_ARG, "unknown epilogue");
  if (epilogue == GPT_EPI_DRELU2 && (!aux || !aligned16(aux)))
    return fail(GPT_ERR_INVALID_ARG, "epilogue needs an aligned aux buffer");
  if (epilogue != GPT_EPI_DRELU2) aux = nullptr;
  if (M < 0 || N < 0 || K < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  const int64_t rowA = op == GPT_GEMM_TN ? M : K, rowB = op == GPT_GEMM_NT ? K : N;
  if (lda < rowA || ldb < rowB || ldc < N) return fail(GPT_ERR_INVALID_ARG, "leading dims too small");
  if (scratch && !aligned16(scratch)) return fail(GPT_ERR_MISALIGNED, "scratch misaligned");
  gk::GemmDesc g{op, M, N, K, A, lda, B, ldb, C, ldc, epilogue, aux,
                 scratch, scratch ? scratch_bytes : 0};
  KERNEL_TRY(gk::gemm(g, (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_fp8_cast_scratch_bytes(void) { return gk::fp8_cast_scratch_bytes(); }

int gpt_k_fp8_cast(const void* x, int64_t rows, int64_t cols, int32_t dtype, int32_t fp8_format,
                   void* q, void* q_t, float* scales, void* scratch, size_t scratch_bytes,
                   hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({x, scratch}))) return st;
  if (!scales || ((uintptr_t)scales & 3u))
    return fail(GPT_ERR_INVALID_ARG, "scales null or not 4-byte aligned");
  if (fp8_format != GPT_FP8_E4M3 && fp8_format != GPT_FP8_E5M2)
    return fail(GPT_ERR_INVALID_ARG, "unknown fp8 format");
  if (!q && !q_t) return fail(GPT_ERR_INVALID_ARG, "no output requested");
  if ((q && !aligned16(q)) || (q_t && !aligned16(q_t)))
    return fail(GPT_ERR_MISALIGNED, "an output is not 16-byte aligned");
  if (rows < 1 || cols < 16 || cols % 16 || (q_t && rows % 16))
    return fail(GPT_ERR_INVALID_ARG, "bad sizes (cols, and rows for q_t, multiples of 16)");
  if (cols > 65535ll * 64 || rows > (1ll << 31) * 64)
    return fail(GPT_ERR_INVALID_ARG, "tensor too large (cols <= 65535 * 64)");
  if (scratch_bytes < gk::fp8_cast_scratch_bytes())
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch needs %zu bytes", gk::fp8_cast_scratch_bytes());
  KERNEL_TRY(gk::fp8_cast(x, rows, cols, (gk::DType)dtype, fp8_format, q, q_t, scales, scratch, s));
  return GPT_OK;
}

size_t gpt_k_gemm_fp8_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 128 || K % 128) return 0;
  return gk::gemm_fp8_scratch_bytes(M, N, K);
}

int gpt_k_gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int32_t fmt_a,
                   const void* B, int64_t ldb, int32_t fmt_b, const float* a_inv_scale,
                   const float* b_inv_scale, void* C, int64_t ldc, int32_t epilogue,
                   void* scratch, size_t scratch_bytes, hipStream_t s) {
  int st;
  if ((st = check_ptrs({A, B, C}))) return st;
  if (!a_inv_scale || !b_inv_scale) return fail(GPT_ERR_INVALID_ARG, "a scale pointer is null");
  if ((fmt_a != GPT_FP8_E4M3 && fmt_a != GPT_FP8_E5M2) ||
      (fmt_b != GPT_FP8_E4M3 && fmt_b != GPT_FP8_E5M2))
    return fail(GPT_ERR_INVALID_ARG, "unknown fp8 format");
  if (epilogue != GPT_EPI_STORE && epilogue != GPT_EPI_F32 && epilogue != GPT_EPI_F32_ACC)
    return fail(GPT_ERR_INVALID_ARG, "epilogue must be STORE, F32 or F32_ACC");
  if (!gk::gemm_fp8_ok(M, N, K, lda, ldb, ldc))
    return fail(GPT_ERR_INVALID_ARG,
                "bad sizes (K a multiple of 128, lda/ldb multiples of 16 and >= K, N and ldc "
                "multiples of 4, operands under 4 GiB)");
  if (scratch && !aligned16(scratch)) return fail(GPT_ERR_MISALIGNED, "scratch misaligned");
  KERNEL_TRY(gk::gemm_fp8(M, N, K, A, lda, fmt_a, B, ldb, fmt_b, a_inv_scale, b_inv_scale, C, ldc,
                          epilogue, scratch, scratch ? scratch_bytes : 0, s));
  return GPT_OK;
}

size_t gpt_k_polar_express_ws_bytes(int32_t batch, int64_t m, int64_t n) {
  if (batch < 1 || batch > 65535 || m < 8 || n < 8 || m % 8 || n % 8) return 0;
  return gk::polar_express_ws_bytes(batch, m, n);
}

int gpt_k_polar_express(const void* g, int32_t batch, int64_t m, int64_t n, int32_t dtype,
                        const float* coeffs, int32_t steps, float eps, void* x_out, void* ws,
                        size_t ws_bytes, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({g, x_out, ws}))) return st;
  if (batch < 1 || batch > 65535) return fail(GPT_ERR_INVALID_ARG, "batch outside [1, 65535]");
  if (m < 8 || n < 8 || m % 8 || n % 8)
    return fail(GPT_ERR_INVALID_ARG, "m and n must be multiples of 8");
  if (steps < 0 || steps > 64 || (steps > 0 && !coeffs))
    return fail(GPT_ERR_INVALID_ARG, "steps outside [0, 64] or coeffs null");
  if (!(eps >= 0.f)) return fail(GPT_ERR_INVALID_ARG, "eps must be >= 0");
  if ((double)batch * m * n * 4 >= 4294967295.0 * 64)
    return fail(GPT_ERR_INVALID_ARG, "batch too large");
  const size_t need = gk::polar_express_ws_bytes(batch, m, n);
  if (ws_bytes < need) return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "ws needs %zu bytes", need);
  KERNEL_TRY(gk::polar_express(g, batch, m, n, (gk::DType)dtype, coeffs, steps, eps, x_out, ws,
                               s));
  return GPT_OK;
}

static int optim_ptrs(std::initializer_list<const void*> ps, int64_t n) {
  int st;
  if ((st = check_ptrs(ps))) return st;
  if (n < 4 || n % 4) return fail(GPT_ERR_INVALID_ARG, "n must be a positive multiple of 4");
  return GPT_OK;
}

int gpt_k_muon_momentum(const float* grad, float* mom, void* u, int64_t n, float beta,
                        int32_t nesterov, int32_t u_dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(u_dtype)) || (st = optim_ptrs({grad, mom, u}, n))) return st;
  if (!(beta >= 0.f && beta < 1.f)) return fail(GPT_ERR_INVALID_ARG, "beta outside [0, 1)");
  KERNEL_TRY(gk::muon_momentum(grad, mom, u, n, beta, nesterov ? 1 : 0, (gk::DType)u_dtype, s));
  return GPT_OK;
}

int gpt_k_muon_update(float* w, const void* x, int64_t n, float lr, float wd, void* w_bf16,
                      hipStream_t s) {
  int st;
  if ((st = optim_ptrs({w, x}, n))) return st;
  if (w_bf16 && !aligned16(w_bf16)) return fail(GPT_ERR_MISALIGNED, "w_bf16 misaligned");
  KERNEL_TRY(gk::muon_update(w, x, n, lr, wd, w_bf16, s));
  return GPT_OK;
}

size_t gpt_k_normuon_scratch_bytes(int64_t rows) {
  return rows < 1 ? 0 : gk::normuon_scratch_bytes(1, rows);
}

int gpt_k_normuon_update(float* w, const void* x, float* v, int64_t rows, int64_t cols,
                         float beta2, float lr, float wd, void* w_bf16, void* scratch,
                         size_t scratch_bytes, hipStream_t s) {
  int st;
  if ((st = check_ptrs({w, x, v, scratch}))) return st;
  if (w_bf16 && !aligned16(w_bf16)) return fail(GPT_ERR_MISALIGNED, "w_bf16 misaligned");
  if (rows < 1 || cols < 8 || cols % 8 || rows * cols >= ((int64_t)1 << 31))
    return fail(GPT_ERR_INVALID_ARG, "rows >= 1, cols a multiple of 8, rows cols < 2^31");
  if (!(beta2 >= 0.f && beta2 < 1.f)) return fail(GPT_ERR_INVALID_ARG, "beta2 outside [0, 1)");
  const size_t need = gk::normuon_scratch_bytes(1, rows);
  if (scratch_bytes < need)
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch needs %zu bytes", need);
  gk::LayerOffsets one{};
  KERNEL_TRY(gk::normuon_update_group(w, x, v, one, 1, rows, cols, beta2, lr, wd, w_bf16,
                                      scratch, s));
  return GPT_OK;
}

int gpt_k_adamw(float* w, const float* grad, float* m, float* v, int64_t n, int32_t step,
                float lr, float beta1, float beta2, float eps, float wd, void* w_bf16,
                hipStream_t s) {
  int st;
  if ((st = optim_ptrs({w, grad, m, v}, n))) return st;
  if (w_bf16 && !aligned16(w_bf16)) return fail(GPT_ERR_MISALIGNED, "w_bf16 misaligned");
  if (step < 1) return fail(GPT_ERR_INVALID_ARG, "step counts from 1");
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f))
    return fail(GPT_ERR_INVALID_ARG, "betas outside [0, 1)");
  KERNEL_TRY(gk::adamw(w, grad, m, v, n, step, lr, beta1, beta2, eps, wd, w_bf16, s));
  return GPT_OK;
}

int gpt_k_resid_mix_fwd(const void* x, const void* x0, void* y, int64_t n, const void* lambdas,
                        int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({x, x0, y}))) return st;
  if (!lambdas) return fail(GPT_ERR_INVALID_ARG, "lambdas is null");
  if (n < 8 || n % 8) return fail(GPT_ERR_INVALID_ARG, "n must be a positive multiple of 8");
  KERNEL_TRY(gk::resid_mix_fwd(x, x0, y, n, lambdas, (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_resid_mix_bwd_scratch_bytes(void) { return gk::resid_mix_bwd_scratch_bytes(); }

int gpt_k_resid_mix_bwd(const void* dy, const void* x, const void* x0, void* dx, void* dx0,
                        int32_t accumulate, int64_t n, const void* lambdas, float* dlambdas,
                        void* scratch, size_t scratch_bytes, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({dy, x, x0, dx0, scratch}))) return st;
  if (dx && !aligned16(dx)) return fail(GPT_ERR_MISALIGNED, "dx misaligned");
  if (!lambdas || !dlambdas) return fail(GPT_ERR_INVALID_ARG, "lambdas or dlambdas is null");
  if (n < 8 || n % 8) return fail(GPT_ERR_INVALID_ARG, "n must be a positive multiple of 8");
  if (scratch_bytes < gk::resid_mix_bwd_scratch_bytes())
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch too small");
  KERNEL_TRY(gk::resid_mix_bwd(dy, x, x0, dx, dx0, accumulate ? 1 : 0, n, lambdas, dlambdas,
                               scratch, (gk::DType)dtype, s));
  return GPT_OK;
}

int gpt_k_smear_fwd(const void* x, int32_t B, int32_t T, int32_t D, const void* w,
                    const void* lambda, void* y, float* gate, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({x, y}))) return st;
  if (!w || !lambda || !gate) return fail(GPT_ERR_INVALID_ARG, "w, lambda or gate is null");
  if (B < 1 || T < 1 || D < 24 || D % 8) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if (x == y) return fail(GPT_ERR_INVALID_ARG, "smear cannot run in place");
  KERNEL_TRY(gk::smear_fwd(x, (int64_t)B * T, T, D, w, lambda, y, gate, (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_smear_bwd_scratch_bytes(void) { return gk::smear_bwd_scratch_bytes(); }

int gpt_k_smear_bwd(const void* dy, const void* x, int32_t B, int32_t T, int32_t D, const void* w,
                    const void* lambda, const float* gate, void* dx, float* dw_dlambda,
                    void* scratch, size_t scratch_bytes, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({dy, x, dx, scratch}))) return st;
  if (!w || !lambda || !gate || !dw_dlambda)
    return fail(GPT_ERR_INVALID_ARG, "w, lambda, gate or dw_dlambda is null");
  if (B < 1 || T < 1 || D < 24 || D % 8) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if (dx == dy || dx == x) return fail(GPT_ERR_INVALID_ARG, "smear backward cannot run in place");
  if (scratch_bytes < gk::smear_bwd_scratch_bytes())
    return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch too small");
  KERNEL_TRY(gk::smear_bwd(dy, x, (int64_t)B * T, T, D, w, lambda, gate, dx, dw_dlambda, scratch,
                           (gk::DType)dtype, s));
  return GPT_OK;
}

int gpt_k_rope_table(float* cs, int32_t T, int32_t hd, float base, hipStream_t s) {
  int st;
  if ((st = check_ptrs({cs}))) return st;
  if (T < 1 || hd < 2 || hd % 2 || !(base > 0.f)) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::rope_table(cs, T, hd, base, s));
  return GPT_OK;
}

static int attn_shape_ok(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd) {
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if (!(hd == 4 || hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128))
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "head_dim %d unsupported", hd);
  return GPT_OK;
}

int gpt_k_rope_qknorm_fwd(void* qkv, float* rq, float* rk, const float* cs, int32_t B, int32_t T,
                          int32_t H, int32_t Hkv, int32_t hd, float eps, int32_t dtype,
                          hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({qkv, rq, rk, cs})) ||
      (st = attn_shape_ok(B, T, H, Hkv, hd)))
    return st;
  KERNEL_TRY(gk::rope_qknorm_fwd(qkv, rq, rk, cs, B, T, H, Hkv, hd, eps, (gk::DType)dtype, s));
  return GPT_OK;
}

int gpt_k_rope_qknorm_bwd(void* dqkv, const void* qkv, const float* rq, const float* rk,
                          const float* cs, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                          int32_t hd, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({dqkv, qkv, rq, rk, cs})) ||
      (st = attn_shape_ok(B, T, H, Hkv, hd)))
    return st;
  KERNEL_TRY(gk::rope_qknorm_bwd(dqkv, qkv, rq, rk, cs, B, T, H, Hkv, hd, (gk::DType)dtype, s));
  return GPT_OK;
}

int gpt_k_attn_fwd(const void* qkv, void* o, float* lse, int32_t B, int32_t T, int32_t H,
                   int32_t Hkv, int32_t hd, int32_t window, int32_t dtype, float score_bound,
                   hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({qkv, o, lse})) ||
      (st = attn_shape_ok(B, T, H, Hkv, hd)))
    return st;
  if (window < 0) return fail(GPT_ERR_INVALID_ARG, "window < 0");
  if (!(score_bound >= 0.f) || !(score_bound < 64.f))
    return fail(GPT_ERR_INVALID_ARG, "score_bound outside [0, 64)");
  KERNEL_TRY(gk::attn_fwd(qkv, o, lse, B, T, H, Hkv, hd, window, (gk::DType)dtype, s,
                          score_bound));
  return GPT_OK;
}

size_t gpt_k_attn_bwd_scratch_bytes(int32_t B, int32_t T, int32_t H, int32_t hd) {
  if (B < 1 || T < 1 || H < 1 || hd < 1) return 0;
  return gk::attn_bwd_scratch_bytes(B, T, H, hd);
}

int gpt_k_attn_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                   void* dqkv, void* scratch, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                   int32_t hd, int32_t window, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({qkv, o, lse, dout, dqkv, scratch})) ||
      (st = attn_shape_ok(B, T, H, Hkv, hd)))
    return st;
  if (window < 0) return fail(GPT_ERR_INVALID_ARG, "window < 0");
  KERNEL_TRY(gk::attn_bwd(qkv, o, lse, dout, dqkv, scratch, B, T, H, Hkv, hd, window,
                          (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_attn_decode_scratch_bytes(int32_t B, int32_t Tq, int32_t H, int32_t Hkv,
                                       int32_t Tmax, int32_t window) {
  if (B < 1 || Tq < 1 || H < 1 || Hkv < 1 || H % Hkv || Tmax < 1 || window < 0) return 0;
  return gk::attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, window);
}

int gpt_k_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_lens, void* o, float* lse, int32_t B, int32_t Tq,
                      int32_t Tmax, int32_t H, int32_t Hkv, int32_t hd, int32_t window,
                      float score_bound, void* scratch, size_t scratch_bytes, int32_t dtype,
                      hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype))) return st;
  if (dtype != GPT_BF16 || hd != 128)
    return fail(GPT_ERR_UNSUPPORTED_CONFIG, "decode attention covers bf16, head_dim 128");
  if (B < 1 || Tq < 1 || Tmax < 1 || H < 1 || Hkv < 1 || H % Hkv)
    return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if ((int64_t)(H / Hkv) * Tq > 1024) return fail(GPT_ERR_INVALID_ARG, "H / Hkv * Tq > 1024");
  if (((int64_t)Tmax + 64) * Hkv > (1ll << 24))
    return fail(GPT_ERR_INVALID_ARG, "(Tmax + 64) * Hkv > 2^24");
  if (B > 65535 || (int64_t)Hkv * ((H / Hkv * Tq + 15) / 16) > 65535)
    return fail(GPT_ERR_INVALID_ARG, "B or Hkv * ceil(H / Hkv * Tq / 16) above 65535");
  if (window < 0) return fail(GPT_ERR_INVALID_ARG, "window < 0");
  if (!(score_bound >= 0.f) || !(score_bound < 64.f))
    return fail(GPT_ERR_INVALID_ARG, "score_bound outside [0, 64)");
  if (!cache_lens || ((uintptr_t)cache_lens & 3u))
    return fail(GPT_ERR_INVALID_ARG, "cache_lens null or misaligned");
  if ((st = check_ptrs({q, k_cache, v_cache, o, lse}))) return st;
  const size_t need = gk::attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, window);
  if (need) {
    if (!scratch) return fail(GPT_ERR_INVALID_ARG, "scratch is null");
    if (!aligned16(scratch)) return fail(GPT_ERR_MISALIGNED, "scratch misaligned");
    if (scratch_bytes < need)
      return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch needs %zu bytes", need);
  }
  KERNEL_TRY(gk::attn_decode(q, k_cache, v_cache, cache_lens, o, lse, B, Tq, Tmax, H, Hkv,
                             window, score_bound, scratch, s));
  return GPT_OK;
}

size_t gpt_k_attn_decode_noalloc_max_scratch(void) { return kDecodeScratchMax; }

int gpt_k_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cache_lens, void* o, float* lse, int32_t B,
                              int32_t Tq, int32_t Tmax, int32_t H, int32_t Hkv, int32_t hd,
                              int32_t window, float score_bound, int32_t dtype, hipStream_t s) {
  // sizes the regular entry rejects give 0 here and are rejected by it below
  const size_t need = gpt_k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, window);
  if (need > kDecodeScratchMax)
    return fail(GPT_ERR_INVALID_ARG,
                "these sizes need %zu bytes of decode scratch; the no-allocation entry holds "
                "%zu (use gpt_k_attn_decode with a caller buffer)", need, kDecodeScratchMax);
  void* p = nullptr;
  if (need) {
    int st = decode_scratch_ptr(&p);
    if (st) return st;
    // the counters start at zero: cleared by a kernel (no memset node, so
    // the call can be captured into a graph)
    const size_t nc = gk::attn_decode_counter_bytes(B, Tq, H, Hkv, Tmax, window);
    KERNEL_TRY(gk::fill_zero(p, (int64_t)nc, s));
  }
  return gpt_k_attn_decode(q, k_cache, v_cache, cache_lens, o, lse, B, Tq, Tmax, H, Hkv, hd,
                           window, score_bound, p, need, dtype, s);
}

int gpt_k_ce(const float* z, const int32_t* tgt, int64_t rows, int32_t V, float* ell, float* lse,
             void* dz, float grad_scale, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({z, tgt, ell, lse}))) return st;
  if (dz && !aligned16(dz)) return fail(GPT_ERR_MISALIGNED, "dz misaligned");
  if (rows < 0 || V < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::ce_rows(z, rows, V, tgt, 1, 1, ell, lse, dz, grad_scale, (gk::DType)dtype, s, 0));
  return GPT_OK;
}

// ---- token embedding and value embedding (kernel-level entries)
int gpt_k_embed_fwd(const int32_t* tokens, int32_t B, int32_t T, const void* wte, int32_t V,
                    int32_t D, void* x, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({tokens, wte, x}))) return st;
  if (B < 1 || T < 1 || V < 1 || D < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::embed_fwd(tokens, B, T, wte, x, D, (gk::DType)dtype, s));
  return GPT_OK;
}

static bool embed_sorted_ok(int32_t D, const void* dx, const float* dW) {
  return D % 4 == 0 && D <= 2048 && aligned16(dx) && aligned16(dW);
}

size_t gpt_k_embed_bwd_scratch_bytes(int32_t B, int32_t T, int32_t V, int32_t D) {
  if (B < 1 || T < 1 || V < 1 || D < 1) return 0;
  return gk::tok_sort_bytes((int64_t)B * T, V, D);
}

int gpt_k_embed_bwd(const int32_t* tokens, int32_t B, int32_t T, const void* dx, int32_t V,
                    int32_t D, float* dwte, int32_t accumulate, void* scratch,
                    size_t scratch_bytes, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({tokens, dx, dwte}))) return st;
  if (B < 1 || T < 1 || V < 1 || D < 1) return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if (accumulate != 0 && accumulate != 1)
    return fail(GPT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  const int64_t N = (int64_t)B * T;
  if (scratch && scratch_bytes >= gk::tok_sort_bytes(N, V, D) && embed_sorted_ok(D, dx, dwte)) {
    KERNEL_TRY(gk::tok_sort(tokens, B, T, V, D, scratch, s));
    KERNEL_TRY(gk::seg_scatter(scratch, N, V, D, dx, D, D, nullptr, 1, D, dwte, accumulate,
                               (gk::DType)dtype, s));
  } else {
    if (!accumulate) KERNEL_TRY(gk::fill_zero(dwte, (int64_t)V * D * 4, s));
    KERNEL_TRY(gk::embed_bwd(tokens, B, T, dx, D, dwte, D, (gk::DType)dtype, s));
  }
  return GPT_OK;
}

int gpt_k_ve_fwd(const int32_t* tokens, int32_t B, int32_t T, const void* h, int32_t D,
                 const void* wg, int32_t C, const void* E, void* qkv, int32_t ldqkv,
                 int32_t voff, float* g, int32_t Hkv, int32_t hd, int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) || (st = check_ptrs({tokens, h, wg, E, qkv, g}))) return st;
  if (B < 1 || T < 1 || D < 1 || C < 1 || C > D || Hkv < 1 || Hkv > 64 || hd < 4 || hd % 4 ||
      voff < 0 || voff + Hkv * hd > ldqkv)
    return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  KERNEL_TRY(gk::ve_fwd(tokens, B, T, h, D, wg, C, E, qkv, ldqkv, voff, g, Hkv, hd,
                        (gk::DType)dtype, s));
  return GPT_OK;
}

size_t gpt_k_ve_bwd_scratch_bytes(int32_t B, int32_t T, int32_t V, int32_t Hkv, int32_t hd,
                                  int32_t C) {
  if (B < 1 || T < 1 || V < 1 || Hkv < 1 || hd < 1 || C < 1) return 0;
  return pad256(gk::ve_wgrad_scratch_bytes(Hkv, C)) +
         gk::tok_sort_bytes((int64_t)B * T, V, Hkv * hd);
}

int gpt_k_ve_bwd(const int32_t* tokens, int32_t B, int32_t T, const void* dqkv, int32_t ldqkv,
                 int32_t voff, const void* E, const float* g, const void* h, int32_t D,
                 int32_t C, int32_t V, int32_t Hkv, int32_t hd, float* vez, float* dE,
                 float* dwg, int32_t accumulate, void* scratch, size_t scratch_bytes,
                 int32_t dtype, hipStream_t s) {
  int st;
  if ((st = dtype_ok(dtype)) ||
      (st = check_ptrs({tokens, dqkv, E, g, h, vez, dE, dwg, scratch})))
    return st;
  if (B < 1 || T < 1 || D < 1 || C < 1 || C > D || V < 1 || Hkv < 1 || Hkv > 64 || hd < 4 ||
      hd % 4 || voff < 0 || voff + Hkv * hd > ldqkv)
    return fail(GPT_ERR_INVALID_ARG, "bad sizes");
  if (accumulate != 0 && accumulate != 1)
    return fail(GPT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  const int64_t N = (int64_t)B * T;
  const int W = Hkv * hd;
  const size_t part = pad256(gk::ve_wgrad_scratch_bytes(Hkv, C));
  if (scratch_bytes < part) return fail(GPT_ERR_WORKSPACE_TOO_SMALL, "scratch too small");
  const gk::DType dt = (gk::DType)dtype;
  const size_t es = dt == gk::BF16 ? 2 : 4;
  const bool sorted = scratch_bytes >= part + gk::tok_sort_bytes(N, V, W) && W % 4 == 0 &&
                      W <= 2048 && ldqkv % 4 == 0 && ((size_t)voff * es) % 16 == 0;
  if (sorted) {
    void* sortws = (char*)scratch + part;
    KERNEL_TRY(gk::tok_sort(tokens, B, T, V, W, sortws, s));
    KERNEL_TRY(gk::ve_vez(tokens, B, T, dqkv, ldqkv, voff, E, g, vez, Hkv, hd, dt, s));
    KERNEL_TRY(gk::seg_scatter(sortws, N, V, W, (const char*)dqkv + voff * es, ldqkv, W, g, Hkv,
                               hd, dE, accumulate, dt, s));
  } else {
    if (!accumulate) KERNEL_TRY(gk::fill_zero(dE, (int64_t)V * W * 4, s));
    KERNEL_TRY(gk::ve_bwd(tokens, B, T, dqkv, ldqkv, voff, E, g, vez, dE, Hkv, hd, dt, s));
  }
  KERNEL_TRY(gk::ve_wgrad(vez, h, D, N, Hkv, C, dwg, accumulate, (float*)scratch, dt, s));
  return GPT_OK;
}

size_t gpt_k_lm_ce_scratch_bytes(int64_t rows, int32_t V) {
  if (rows < 1 || V < 256 || V % 256) return 0;
  return pad256(gk::lm_ce_stats_bytes(rows, V)) + pad256((size_t)rows * 4);
}

int gpt_k_lm_ce(const void* h, const void* w, const int32_t* tgt, int64_t rows, int32_t D,
                int32_t V, float* ell, float* lse, void* dz, float grad_scale, void* scratch,
                hipStream_t s) {
  int st;
  if ((st = check_ptrs({h, w, tgt, ell, lse, scratch}))) return st;
  if (dz && !aligned16(dz)) return fail(GPT_ERR_MISALIGNED, "dz not 16-byte aligned");
  if (!gk::lm_ce_fused_ok(rows, V, D))
    return fail(GPT_ERR_INVALID_ARG,
                "fused lm_head/CE needs rows >= 1, V a multiple of 256 (<= 262144), D a "
                "multiple of 64 and operands under 4 GiB");
  float* stats = (float*)scratch;
  float* zt = (float*)((char*)scratch + pad256(gk::lm_ce_stats_bytes(rows, V)));
  KERNEL_TRY(gk::lm_ce_gemm(h, rows, D, w, V, dz, stats, zt, tgt, 1, 1, s));
  KERNEL_TRY(gk::ce_fix(stats, zt, rows, V, tgt, 1, 1, ell, lse, dz, dz, grad_scale, s));
  return GPT_OK;
}

}  // extern "C"
