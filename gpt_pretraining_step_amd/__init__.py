"""MI355X (gfx950) GPT training step: thin Python binding of libgptstep.so.

Argument marshalling only.  Every step of the forward, backward and
evaluation runs in the library's HIP kernels; torch provides device memory
(tensors) and the current stream.  If the library is not built this module
raises on first use: there is no CPU fallback.

The C ABI and its conventions are documented in include/gpt_step.h.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptstep.so")

F32, BF16 = 0, 1
MODE_TRAIN, MODE_EVAL = 0, 1
GEMM_NT, GEMM_NN, GEMM_TN = 0, 1, 2
EPI_STORE, EPI_RESADD, EPI_RELU2, EPI_DRELU2, EPI_F32, EPI_F32_ACC = range(6)
P_WTE, P_WQKV, P_WO, P_WFC, P_WPROJ, P_VE, P_WG, P_WLM, P_EXTRAS = range(9)
(WS_ELL, WS_LOSS, WS_NONFINITE, WS_X_H, WS_X_QKV, WS_X_O, WS_X_LSE, WS_X_H2,
 WS_X_A, WS_X_HF, WS_BAD_TOKENS) = range(11)


class GptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gpt_step status {status}: {msg}")
        self.status = status


class GptConfig(C.Structure):
    _fields_ = [
        ("n_layer", C.c_int32), ("d_model", C.c_int32), ("n_head", C.c_int32),
        ("n_kv_head", C.c_int32), ("head_dim", C.c_int32), ("vocab", C.c_int32),
        ("seq_len", C.c_int32), ("batch", C.c_int32), ("mlp_mult", C.c_int32),
        ("ve_gate_channels", C.c_int32), ("window_pattern", C.c_char * 16),
        ("window_short", C.c_int32), ("window_long", C.c_int32),
        ("ve_every_odd", C.c_int32), ("rope_base", C.c_float),
        ("norm_eps", C.c_float), ("dtype", C.c_int32),
        ("resid_lambdas", C.c_int32), ("smear", C.c_int32), ("backout", C.c_int32),
        ("backout_layer", C.c_int32), ("check_tokens", C.c_int32), ("one_stream", C.c_int32),
    ]


class OptimHparams(C.Structure):
    _fields_ = [
        ("muon_lr", C.c_float), ("muon_momentum", C.c_float), ("muon_wd", C.c_float),
        ("muon_nesterov", C.c_int32), ("ns_steps", C.c_int32), ("ns_coeffs", C.c_float * 48),
        ("ns_eps", C.c_float), ("adam_lr_embed", C.c_float), ("adam_lr_head", C.c_float),
        ("adam_lr_gate", C.c_float), ("adam_beta1", C.c_float), ("adam_beta2", C.c_float),
        ("adam_eps", C.c_float), ("adam_wd", C.c_float),
        ("normuon", C.c_int32), ("normuon_beta2", C.c_float),
    ]


def make_optim_hparams(coeffs, muon_lr=0.02, muon_momentum=0.95, muon_wd=0.0, nesterov=True,
                       ns_eps=1e-7, adam_lr_embed=0.2, adam_lr_head=0.004, adam_lr_gate=0.02,
                       beta1=0.8, beta2=0.95, eps=1e-10, adam_wd=0.0, normuon=False,
                       normuon_beta2=0.95) -> OptimHparams:
    h = OptimHparams()
    h.muon_lr, h.muon_momentum, h.muon_wd = muon_lr, muon_momentum, muon_wd
    h.muon_nesterov, h.ns_steps = int(nesterov), len(coeffs)
    flat = [float(v) for t in coeffs for v in t]
    for i, v in enumerate(flat):
        h.ns_coeffs[i] = v
    h.ns_eps = ns_eps
    h.adam_lr_embed, h.adam_lr_head, h.adam_lr_gate = adam_lr_embed, adam_lr_head, adam_lr_gate
    h.adam_beta1, h.adam_beta2, h.adam_eps, h.adam_wd = beta1, beta2, eps, adam_wd
    h.normuon, h.normuon_beta2 = int(normuon), normuon_beta2
    return h


def make_config(d: dict) -> GptConfig:
    """A GptConfig from a dict with the struct's field names.  The model
    extras default to off; backout_layer -1 (or absent) means no backout."""
    c = GptConfig()
    d = dict(d)
    d.setdefault("resid_lambdas", 0)
    d.setdefault("smear", 0)
    d.setdefault("check_tokens", 0)
    d.setdefault("one_stream", 0)
    bl = int(d.get("backout_layer", -1))
    d["backout"], d["backout_layer"] = (1, bl) if bl >= 0 else (0, 0)
    for name, _ in GptConfig._fields_:
        v = d[name]
        if name == "window_pattern":
            v = (v or "").encode()
        setattr(c, name, v)
    return c


_lib = None
_vp, _i32, _i64, _f32, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_cfgp = C.POINTER(GptConfig)

_SIGS = {
    "gpt_validate_config": (C.c_int, [_cfgp]),
    "gpt_param_count": (_i64, [_cfgp]),
    "gpt_param_offset": (_i64, [_cfgp, C.c_int, C.c_int]),
    "gpt_workspace_bytes": (_sz, [_cfgp, C.c_int]),
    "gpt_ws_offset": (_i64, [_cfgp, C.c_int, C.c_int]),
    "gpt_step_fwd": (C.c_int, [_cfgp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "gpt_step_bwd": (C.c_int, [_cfgp, _vp, _vp, _vp, _sz, _vp, C.c_int, _vp]),
    "gpt_eval_bpb": (C.c_int, [_cfgp, _vp, _vp, _i64, _vp, _vp, _sz, _vp, _vp]),
    "gpt_status_string": (C.c_char_p, [C.c_int]),
    "gpt_last_error": (C.c_char_p, []),
    "gpt_k_rmsnorm_fwd": (C.c_int, [_vp, _vp, _vp, _i64, _i32, _f32, _i32, _vp]),
    "gpt_k_rmsnorm_bwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp]),
    "gpt_k_gemm_scratch_bytes": (_sz, [_i64, _i64, _i64]),
    "gpt_k_gemm": (C.c_int, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                             _i32, _vp, _vp, _sz, _i32, _vp]),
    "gpt_k_rope_table": (C.c_int, [_vp, _i32, _i32, _f32, _vp]),
    "gpt_k_rope_qknorm_fwd": (C.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _f32, _i32, _vp]),
    "gpt_k_rope_qknorm_bwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _vp]),
    "gpt_k_attn_fwd": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                 _vp]),
    "gpt_k_attn_bwd_scratch_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "gpt_k_attn_bwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _vp]),
    "gpt_k_attn_decode_scratch_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "gpt_k_attn_decode": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _f32, _vp, _sz, _i32, _vp]),
    "gpt_k_attn_decode_noalloc_max_scratch": (_sz, []),
    "gpt_k_attn_decode_noalloc": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "gpt_k_fp8_cast_scratch_bytes": (_sz, []),
    "gpt_k_fp8_cast": (C.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_k_gemm_fp8_scratch_bytes": (_sz, [_i64, _i64, _i64]),
    "gpt_k_gemm_fp8": (C.c_int, [_i64, _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _vp, _vp,
                                 _vp, _i64, _i32, _vp, _sz, _vp]),
    "gpt_k_polar_express_ws_bytes": (_sz, [_i32, _i64, _i64]),
    "gpt_k_polar_express": (C.c_int, [_vp, _i32, _i64, _i64, _i32, _vp, _i32, _f32, _vp, _vp,
                                      _sz, _vp]),
    "gpt_k_muon_momentum": (C.c_int, [_vp, _vp, _vp, _i64, _f32, _i32, _i32, _vp]),
    "gpt_k_muon_update": (C.c_int, [_vp, _vp, _i64, _f32, _f32, _vp, _vp]),
    "gpt_k_normuon_scratch_bytes": (_sz, [_i64]),
    "gpt_k_normuon_update": (C.c_int, [_vp, _vp, _vp, _i64, _i64, _f32, _f32, _f32, _vp, _vp,
                                       _sz, _vp]),
    "gpt_k_adamw": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _f32, _f32, _f32, _f32, _f32, _vp,
                              _vp]),
    "gpt_k_resid_mix_fwd": (C.c_int, [_vp, _vp, _vp, _i64, _vp, _i32, _vp]),
    "gpt_k_resid_mix_bwd_scratch_bytes": (_sz, []),
    "gpt_k_resid_mix_bwd": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz,
                                      _i32, _vp]),
    "gpt_k_smear_fwd": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp]),
    "gpt_k_smear_bwd_scratch_bytes": (_sz, []),
    "gpt_k_smear_bwd": (C.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                  _i32, _vp]),
    "gpt_optim_ws_bytes": (_sz, [_vp]),
    "gpt_optim_step": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gpt_k_ce": (C.c_int, [_vp, _vp, _i64, _i32, _vp, _vp, _vp, _f32, _i32, _vp]),
    "gpt_k_lm_ce_scratch_bytes": (_sz, [_i64, _i32]),
    "gpt_k_embed_fwd": (C.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _vp, _i32, _vp]),
    "gpt_k_embed_bwd_scratch_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "gpt_k_embed_bwd": (C.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _sz, _i32,
                                  _vp]),
    "gpt_k_ve_fwd": (C.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp,
                               _i32, _i32, _i32, _vp]),
    "gpt_k_ve_bwd_scratch_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "gpt_k_ve_bwd": (C.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                               _i32, _i32, _vp, _vp, _vp, _i32, _vp, _sz, _i32, _vp]),
    "gpt_k_lm_ce": (C.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _f32, _vp, _vp]),
    "gpt_prof_start": (C.c_int, [_i32]),
    "gpt_prof_stop": (C.c_int, []),
    "gpt_prof_count": (_i32, []),
    "gpt_prof_record": (C.c_int, [_i32, C.c_char_p, _sz, C.POINTER(C.c_float),
                                  C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "gpt_prof_clear": (None, []),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gpt_pretraining_step_amd.build` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _check(status: int):
    if status != 0:
        raise GptError(status, lib().gpt_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


# ------------------------------------------------------------ model level
def validate_config(cfg: GptConfig) -> int:
    return lib().gpt_validate_config(C.byref(cfg))


def param_count(cfg: GptConfig) -> int:
    n = lib().gpt_param_count(C.byref(cfg))
    if n < 0:
        _check(int(n))
    return int(n)


def param_offset(cfg: GptConfig, which: int, layer: int = 0) -> int:
    n = lib().gpt_param_offset(C.byref(cfg), which, layer)
    if n < -1:
        _check(int(n))
    return int(n)


def workspace_bytes(cfg: GptConfig, mode: int = MODE_TRAIN) -> int:
    n = lib().gpt_workspace_bytes(C.byref(cfg), mode)
    if n == 0:
        raise GptError(-1, lib().gpt_last_error().decode())
    return int(n)


def ws_offset(cfg: GptConfig, which: int, layer: int = 0) -> int:
    n = lib().gpt_ws_offset(C.byref(cfg), which, layer)
    if n < -1:
        _check(int(n))
    return int(n)


def step_fwd(cfg, params, tokens, ws, loss, stream=None):
    _check(lib().gpt_step_fwd(C.byref(cfg), _ptr(params), _ptr(tokens), _ptr(ws),
                              ws.numel() * ws.element_size(), _ptr(loss), _stream(stream)))


def step_bwd(cfg, params, tokens, ws, grads, accumulate=False, stream=None):
    _check(lib().gpt_step_bwd(C.byref(cfg), _ptr(params), _ptr(tokens), _ptr(ws),
                              ws.numel() * ws.element_size(), _ptr(grads),
                              1 if accumulate else 0, _stream(stream)))


def eval_bpb(cfg, params, tokens, token_bytes, ws, out, stream=None):
    _check(lib().gpt_eval_bpb(C.byref(cfg), _ptr(params), _ptr(tokens), tokens.shape[0],
                              _ptr(token_bytes), _ptr(ws), ws.numel() * ws.element_size(),
                              _ptr(out), _stream(stream)))


# ------------------------------------------------------------ kernel level
def k_rmsnorm_fwd(x, y, r, rows, dim, eps, dtype, stream=None):
    _check(lib().gpt_k_rmsnorm_fwd(_ptr(x), _ptr(y), _ptr(r), rows, dim, eps, dtype,
                                   _stream(stream)))


def k_rmsnorm_bwd(dy, y, r, dres, dx, rows, dim, dtype, stream=None):
    _check(lib().gpt_k_rmsnorm_bwd(_ptr(dy), _ptr(y), _ptr(r), _ptr(dres), _ptr(dx), rows, dim,
                                   dtype, _stream(stream)))


def k_gemm_scratch_bytes(M, N, K):
    return int(lib().gpt_k_gemm_scratch_bytes(M, N, K))


def k_gemm(op, M, N, K, A, lda, B, ldb, Cm, ldc, epi, aux, dtype, stream=None, scratch=None):
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    _check(lib().gpt_k_gemm(op, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(Cm), ldc, epi,
                            _ptr(aux), _ptr(scratch), nbytes, dtype, _stream(stream)))


def k_rope_table(cs, T, hd, base, stream=None):
    _check(lib().gpt_k_rope_table(_ptr(cs), T, hd, base, _stream(stream)))


def k_rope_qknorm_fwd(qkv, rq, rk, cs, B, T, H, Hkv, hd, eps, dtype, stream=None):
    _check(lib().gpt_k_rope_qknorm_fwd(_ptr(qkv), _ptr(rq), _ptr(rk), _ptr(cs), B, T, H, Hkv,
                                       hd, eps, dtype, _stream(stream)))


def k_rope_qknorm_bwd(dqkv, qkv, rq, rk, cs, B, T, H, Hkv, hd, dtype, stream=None):
    _check(lib().gpt_k_rope_qknorm_bwd(_ptr(dqkv), _ptr(qkv), _ptr(rq), _ptr(rk), _ptr(cs), B,
                                       T, H, Hkv, hd, dtype, _stream(stream)))


def k_attn_fwd(qkv, o, lse, B, T, H, Hkv, hd, window, dtype, stream=None, score_bound=0.0):
    _check(lib().gpt_k_attn_fwd(_ptr(qkv), _ptr(o), _ptr(lse), B, T, H, Hkv, hd, window, dtype,
                                score_bound, _stream(stream)))


def k_attn_bwd_scratch_bytes(B, T, H, hd):
    return int(lib().gpt_k_attn_bwd_scratch_bytes(B, T, H, hd))


def k_attn_bwd(qkv, o, lse, dout, dqkv, scratch, B, T, H, Hkv, hd, window, dtype, stream=None):
    _check(lib().gpt_k_attn_bwd(_ptr(qkv), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dqkv),
                                _ptr(scratch), B, T, H, Hkv, hd, window, dtype, _stream(stream)))


def k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, window):
    return int(lib().gpt_k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, window))


def k_attn_decode(q, k_cache, v_cache, cache_lens, o, lse, B, Tq, Tmax, H, Hkv, hd, window,
                  score_bound, scratch, dtype, stream=None):
    nb = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(lib().gpt_k_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens),
                                   _ptr(o), _ptr(lse), B, Tq, Tmax, H, Hkv, hd, window,
                                   score_bound, _ptr(scratch), nb, dtype, _stream(stream)))


def k_attn_decode_noalloc_max_scratch():
    return int(lib().gpt_k_attn_decode_noalloc_max_scratch())


def k_attn_decode_noalloc(q, k_cache, v_cache, cache_lens, o, lse, B, Tq, Tmax, H, Hkv, hd,
                          window, score_bound, dtype, stream=None):
    _check(lib().gpt_k_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(cache_lens), _ptr(o), _ptr(lse), B, Tq, Tmax,
                                           H, Hkv, hd, window, score_bound, dtype,
                                           _stream(stream)))


FP8_E4M3, FP8_E5M2 = 0, 1


def k_fp8_cast_scratch_bytes():
    return int(lib().gpt_k_fp8_cast_scratch_bytes())


def k_fp8_cast(x, rows, cols, dtype, fmt, q, q_t, scales, scratch, stream=None):
    nb = scratch.numel() * scratch.element_size()
    _check(lib().gpt_k_fp8_cast(_ptr(x), rows, cols, dtype, fmt, _ptr(q), _ptr(q_t),
                                _ptr(scales), _ptr(scratch), nb, _stream(stream)))


def k_gemm_fp8_scratch_bytes(M, N, K):
    return int(lib().gpt_k_gemm_fp8_scratch_bytes(M, N, K))


def k_gemm_fp8(M, N, K, A, lda, fmt_a, B, ldb, fmt_b, a_inv, b_inv, C, ldc, epilogue,
               scratch=None, stream=None):
    nb = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(lib().gpt_k_gemm_fp8(M, N, K, _ptr(A), lda, fmt_a, _ptr(B), ldb, fmt_b, _ptr(a_inv),
                                _ptr(b_inv), _ptr(C), ldc, epilogue, _ptr(scratch), nb,
                                _stream(stream)))


def k_polar_express_ws_bytes(m, n, batch=1):
    return int(lib().gpt_k_polar_express_ws_bytes(batch, m, n))


def k_polar_express(g, m, n, dtype, coeffs, eps, x_out, ws, batch=1, stream=None):
    """coeffs: a sequence of (a, b, c) tuples (host)."""
    flat = [float(v) for t in coeffs for v in t]
    arr = (C.c_float * max(1, len(flat)))(*flat)
    _check(lib().gpt_k_polar_express(_ptr(g), batch, m, n, dtype, C.cast(arr, C.c_void_p),
                                     len(coeffs), eps, _ptr(x_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def k_muon_momentum(grad, mom, u, n, beta, nesterov, u_dtype, stream=None):
    _check(lib().gpt_k_muon_momentum(_ptr(grad), _ptr(mom), _ptr(u), n, beta, int(nesterov),
                                     u_dtype, _stream(stream)))


def k_muon_update(w, x, n, lr, wd, w_bf16=None, stream=None):
    _check(lib().gpt_k_muon_update(_ptr(w), _ptr(x), n, lr, wd, _ptr(w_bf16), _stream(stream)))


def k_adamw(w, grad, m, v, n, step, lr, beta1, beta2, eps, wd, w_bf16=None, stream=None):
    _check(lib().gpt_k_adamw(_ptr(w), _ptr(grad), _ptr(m), _ptr(v), n, step, lr, beta1, beta2,
                             eps, wd, _ptr(w_bf16), _stream(stream)))


def k_normuon_scratch_bytes(rows) -> int:
    return int(lib().gpt_k_normuon_scratch_bytes(rows))


def k_normuon_update(w, x, v, rows, cols, beta2, lr, wd, scratch, w_bf16=None, stream=None):
    _check(lib().gpt_k_normuon_update(_ptr(w), _ptr(x), _ptr(v), rows, cols, beta2, lr, wd,
                                      _ptr(w_bf16), _ptr(scratch), scratch.numel(),
                                      _stream(stream)))


def k_resid_mix_fwd(x, x0, y, n, lambdas, dtype, stream=None):
    _check(lib().gpt_k_resid_mix_fwd(_ptr(x), _ptr(x0), _ptr(y), n, _ptr(lambdas), dtype,
                                     _stream(stream)))


def k_resid_mix_bwd(dy, x, x0, dx, dx0, accumulate, n, lambdas, dlambdas, scratch, dtype,
                    stream=None):
    _check(lib().gpt_k_resid_mix_bwd(_ptr(dy), _ptr(x), _ptr(x0), _ptr(dx), _ptr(dx0),
                                     int(accumulate), n, _ptr(lambdas), _ptr(dlambdas),
                                     _ptr(scratch), scratch.numel() * scratch.element_size(),
                                     dtype, _stream(stream)))


def k_smear_fwd(x, B, T, D, w, lam, y, gate, dtype, stream=None):
    _check(lib().gpt_k_smear_fwd(_ptr(x), B, T, D, _ptr(w), _ptr(lam), _ptr(y), _ptr(gate),
                                 dtype, _stream(stream)))


def k_smear_bwd(dy, x, B, T, D, w, lam, gate, dx, dw_dlam, scratch, dtype, stream=None):
    _check(lib().gpt_k_smear_bwd(_ptr(dy), _ptr(x), B, T, D, _ptr(w), _ptr(lam), _ptr(gate),
                                 _ptr(dx), _ptr(dw_dlam), _ptr(scratch),
                                 scratch.numel() * scratch.element_size(), dtype,
                                 _stream(stream)))


def optim_ws_bytes(cfg: GptConfig) -> int:
    return int(lib().gpt_optim_ws_bytes(C.byref(cfg)))


def optim_step(cfg: GptConfig, hp: OptimHparams, step, master, params, grads, state1, state2,
               ws, stream=None):
    _check(lib().gpt_optim_step(C.byref(cfg), C.byref(hp), step, _ptr(master), _ptr(params),
                                _ptr(grads), _ptr(state1), _ptr(state2), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def k_embed_fwd(tokens, B, T, wte, V, D, x, dtype, stream=None):
    _check(lib().gpt_k_embed_fwd(_ptr(tokens), B, T, _ptr(wte), V, D, _ptr(x), dtype,
                                 _stream(stream)))


def k_embed_bwd_scratch_bytes(B, T, V, D):
    return int(lib().gpt_k_embed_bwd_scratch_bytes(B, T, V, D))


def k_embed_bwd(tokens, B, T, dx, V, D, dwte, accumulate, scratch, dtype, stream=None):
    nb = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(lib().gpt_k_embed_bwd(_ptr(tokens), B, T, _ptr(dx), V, D, _ptr(dwte), accumulate,
                                 _ptr(scratch), nb, dtype, _stream(stream)))


def k_ve_fwd(tokens, B, T, h, D, wg, C_, E, qkv, ldqkv, voff, g, Hkv, hd, dtype, stream=None):
    _check(lib().gpt_k_ve_fwd(_ptr(tokens), B, T, _ptr(h), D, _ptr(wg), C_, _ptr(E), _ptr(qkv),
                              ldqkv, voff, _ptr(g), Hkv, hd, dtype, _stream(stream)))


def k_ve_bwd_scratch_bytes(B, T, V, Hkv, hd, C_):
    return int(lib().gpt_k_ve_bwd_scratch_bytes(B, T, V, Hkv, hd, C_))


def k_ve_bwd(tokens, B, T, dqkv, ldqkv, voff, E, g, h, D, C_, V, Hkv, hd, vez, dE, dwg,
             accumulate, scratch, dtype, stream=None):
    nb = scratch.numel() * scratch.element_size()
    _check(lib().gpt_k_ve_bwd(_ptr(tokens), B, T, _ptr(dqkv), ldqkv, voff, _ptr(E), _ptr(g),
                              _ptr(h), D, C_, V, Hkv, hd, _ptr(vez), _ptr(dE), _ptr(dwg),
                              accumulate, _ptr(scratch), nb, dtype, _stream(stream)))


def k_lm_ce_scratch_bytes(rows, V):
    return int(lib().gpt_k_lm_ce_scratch_bytes(rows, V))


def k_lm_ce(h, w, tgt, rows, D, V, ell, lse, dz, grad_scale, scratch, stream=None):
    _check(lib().gpt_k_lm_ce(_ptr(h), _ptr(w), _ptr(tgt), rows, D, V, _ptr(ell), _ptr(lse),
                             _ptr(dz), grad_scale, _ptr(scratch), _stream(stream)))


def k_ce(z, tgt, rows, V, ell, lse, dz, grad_scale, dtype, stream=None):
    _check(lib().gpt_k_ce(_ptr(z), _ptr(tgt), rows, V, _ptr(ell), _ptr(lse), _ptr(dz),
                          grad_scale, dtype, _stream(stream)))


# ------------------------------------------------------- launch recording
def prof_start(capacity: int = 65536):
    """Record every kernel launch (two HIP events each on its own stream)."""
    _check(lib().gpt_prof_start(capacity))


def prof_stop() -> bool:
    """Stop recording; True if launches beyond the capacity went unrecorded."""
    return bool(lib().gpt_prof_stop())


def prof_records():
    """[(kernel name, ms, flops, bytes)] of the recorded launches, in order
    (waits for them to finish)."""
    L = lib()
    buf = C.create_string_buffer(1024)
    ms, fl, by = C.c_float(), C.c_double(), C.c_double()
    out = []
    for i in range(int(L.gpt_prof_count())):
        _check(L.gpt_prof_record(i, buf, len(buf), C.byref(ms), C.byref(fl), C.byref(by)))
        out.append((buf.value.decode(), float(ms.value), float(fl.value), float(by.value)))
    return out


def prof_clear():
    lib().gpt_prof_clear()

