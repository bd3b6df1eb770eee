"""Host-side tests of the C ABI (no GPU work is enqueued by any of them).

The library must load, export every function include/gpt_step.h declares,
agree with the oracle on parameter layout, and reject bad arguments with
distinct status codes before anything reaches the GPU.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import gptinputs as gi
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

G = pytest.importorskip("gpt_pretraining_step_amd")
if not os.path.exists(G.LIB_PATH):
    pytest.skip("libgptstep.so not built", allow_module_level=True)


def header_functions():
    src = open(os.path.join(ROOT, "include", "gpt_step.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = G.lib()
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(G.exported_symbols())


_EXTRAS = dict(resid_lambdas=1, smear=1, backout_layer=2)


@pytest.mark.parametrize("name", list(gi.PRESETS) + ["d4+extras", "d12+backout"])
def test_param_layout_matches_oracle(name):
    if name == "d4+extras":
        d = gi.preset("d4", **_EXTRAS)
    elif name == "d12+backout":
        d = gi.preset("d12", backout_layer=5)
    else:
        d = gi.preset(name)
    c = G.make_config(d)
    assert G.param_count(c) == O.param_count(d)
    off, layers = 0, {}
    for tname, shape in O.param_layout(d):
        layers[tname] = off
        off += int(np.prod(shape))
    assert G.param_offset(c, G.P_WTE) == layers["wte"]
    assert G.param_offset(c, G.P_WLM) == layers["wlm"]
    for l in range(d["n_layer"]):
        assert G.param_offset(c, G.P_WQKV, l) == layers[f"l{l}.wqkv"]
        assert G.param_offset(c, G.P_WO, l) == layers[f"l{l}.wo"]
        assert G.param_offset(c, G.P_WFC, l) == layers[f"l{l}.wfc"]
        assert G.param_offset(c, G.P_WPROJ, l) == layers[f"l{l}.wproj"]
        assert G.param_offset(c, G.P_VE, l) == layers.get(f"l{l}.ve", -1)
        assert G.param_offset(c, G.P_WG, l) == layers.get(f"l{l}.wg", -1)
    assert G.param_offset(c, G.P_EXTRAS) == layers.get("extras", -1)
    if "extras" in layers:
        assert O.extras_slots(d) == dict(smear_w=2 * d["n_layer"], smear_lambda=2 * d["n_layer"] + 24,
                                         backout=2 * d["n_layer"] + 25,
                                         size=G.param_count(c) - layers["extras"])


def test_workspace_sizes():
    for name in gi.PRESETS:
        c = G.make_config(gi.preset(name))
        tr, ev = G.workspace_bytes(c, G.MODE_TRAIN), G.workspace_bytes(c, G.MODE_EVAL)
        assert tr > ev > 0
        assert tr % 256 == 0
        # the extras add the saved streams (x0, the kept stream, one per block
        # after the first, their gradients, the smear input)
        ce = G.make_config(gi.preset(name, **_EXTRAS, d_model=max(32, gi.preset(name)["d_model"])))
        if gi.preset(name)["d_model"] >= 32:
            d = gi.preset(name)
            xb = d["batch"] * d["seq_len"] * d["d_model"] * (2 if d["dtype"] == G.BF16 else 4)
            assert G.workspace_bytes(ce, G.MODE_TRAIN) - tr >= (d["n_layer"] + 5) * xb
            assert G.workspace_bytes(ce, G.MODE_EVAL) - ev >= 3 * xb
    # d24 training state fits one 288 GB device with room to spare
    assert G.workspace_bytes(G.make_config(gi.preset("d24"))) < 64 << 30


def _bad(**kw):
    return G.make_config(dict(gi.preset("d4"), **kw))


@pytest.mark.parametrize("kw,status", [
    (dict(n_head=3, n_kv_head=2), -2),
    (dict(head_dim=96), -2),
    (dict(head_dim=0), -2),
    (dict(window_pattern="SXL"), -1),
    (dict(dtype=7), -1),
    (dict(vocab=1), -1),
    (dict(n_layer=0), -1),
    (dict(norm_eps=0.0), -1),
    (dict(ve_gate_channels=0), -1),
    (dict(ve_gate_channels=4096), -1),
    (dict(window_short=-1), -1),
    (dict(backout_layer=4), -1),
    (dict(smear=2), -1),
    (dict(check_tokens=2), -1),
    (dict(one_stream=3), -1),
    (dict(resid_lambdas=1, d_model=252, n_head=2, head_dim=128), -2),
    (dict(smear=1, d_model=16, n_head=2, head_dim=8, ve_gate_channels=8), -2),
])
def test_invalid_configs_rejected(kw, status):
    c = _bad(**kw)
    assert G.validate_config(c) == status
    assert G.lib().gpt_param_count(C.byref(c)) == status
    assert G.lib().gpt_workspace_bytes(C.byref(c), 0) == 0
    assert len(G.lib().gpt_last_error()) > 0


def _call_fwd(c, params, tokens, ws, ws_bytes, loss):
    return G.lib().gpt_step_fwd(C.byref(c), params, tokens, ws, ws_bytes, loss, None)


def test_entry_points_reject_bad_pointers_before_launch():
    c = G.make_config(gi.preset("tiny"))
    need = G.workspace_bytes(c)
    A = C.c_void_p(0x1000)          # never dereferenced: validation fails first
    assert _call_fwd(c, None, A, A, need, A) == -1
    assert _call_fwd(c, C.c_void_p(0x1004), A, A, need, A) == -4
    assert _call_fwd(c, A, A, A, need - 1, A) == -3
    assert G.lib().gpt_step_bwd(C.byref(c), A, A, A, need, A, 2, None) == -1
    assert G.lib().gpt_step_bwd(C.byref(c), A, A, A, need, None, 0, None) == -1
    assert G.lib().gpt_eval_bpb(C.byref(c), A, A, 0, A, A, G.workspace_bytes(c, 1), A, None) == -1
    assert G.lib().gpt_eval_bpb(C.byref(c), A, A, 3, A, A, 16, A, None) == -3
    bad = _bad(n_head=3, n_kv_head=2)
    assert _call_fwd(bad, A, A, A, need, A) == -2
    # kernel entries
    L = G.lib()
    assert L.gpt_k_gemm(5, 4, 4, 4, A, 4, A, 4, A, 4, 0, None, None, 0, 1, None) == -1
    assert L.gpt_k_gemm(0, 4, 4, 4, A, 2, A, 4, A, 4, 0, None, None, 0, 1, None) == -1
    assert L.gpt_k_gemm(0, 4, 4, 4, A, 4, A, 4, A, 4, 3, None, None, 0, 1, None) == -1
    assert L.gpt_k_gemm(0, 4, 4, 4, A, 4, A, 4, A, 4, 0, None, C.c_void_p(0x1008), 64, 1, None) == -4
    assert L.gpt_k_attn_fwd(A, A, A, 1, 8, 3, 2, 128, 4, 1, 0.0, None) == -1
    assert L.gpt_k_attn_fwd(A, A, A, 1, 8, 2, 2, 96, 4, 1, 0.0, None) == -2
    assert L.gpt_k_attn_fwd(A, A, A, 1, 8, 2, 2, 128, 4, 1, -1.0, None) == -1
    assert L.gpt_k_attn_fwd(A, A, A, 1, 8, 2, 2, 128, 4, 1, float("nan"), None) == -1
    assert L.gpt_k_rmsnorm_fwd(A, C.c_void_p(0x1002), A, 4, 8, 1e-5, 1, None) == -4
    # fp8 cast: x, rows, cols, dtype, fmt, q, q_t, scales, scratch, bytes
    cs = L.gpt_k_fp8_cast_scratch_bytes()
    assert cs >= 4096
    assert L.gpt_k_fp8_cast(A, 64, 64, 1, 2, A, None, A, A, cs, None) == -1
    assert L.gpt_k_fp8_cast(A, 64, 64, 1, 0, None, None, A, A, cs, None) == -1
    assert L.gpt_k_fp8_cast(A, 64, 40, 1, 0, A, None, A, A, cs, None) == -1
    assert L.gpt_k_fp8_cast(A, 70, 64, 1, 0, None, A, A, A, cs, None) == -1
    assert L.gpt_k_fp8_cast(A, 64, 64, 1, 0, A, None, A, A, cs - 1, None) == -3
    assert L.gpt_k_fp8_cast(A, 64, 64, 1, 0, C.c_void_p(0x1001), None, A, A, cs, None) == -4
    # fp8 gemm: M, N, K, A, lda, fa, B, ldb, fb, ai, bi, C, ldc, epi, scratch, bytes
    g8 = L.gpt_k_gemm_fp8
    assert g8(64, 64, 100, A, 128, 0, A, 128, 0, A, A, A, 64, 0, None, 0, None) == -1
    assert g8(64, 64, 128, A, 136, 0, A, 128, 0, A, A, A, 64, 0, None, 0, None) == -1
    assert g8(64, 64, 128, A, 128, 0, A, 128, 0, A, A, A, 64, 1, None, 0, None) == -1
    assert g8(64, 64, 128, A, 128, 3, A, 128, 0, A, A, A, 64, 0, None, 0, None) == -1
    assert g8(64, 64, 128, A, 128, 0, A, 128, 0, None, A, A, 64, 0, None, 0, None) == -1
    assert g8(64, 62, 128, A, 128, 0, A, 128, 0, A, A, A, 64, 0, None, 0, None) == -1
    assert L.gpt_k_gemm_fp8_scratch_bytes(256, 256, 8192) > 0
    assert L.gpt_k_gemm_fp8_scratch_bytes(256, 256, 100) == 0
    # Newton-Schulz: g, batch, m, n, dtype, coeffs, steps, eps, x_out, ws, ws_bytes
    ns = L.gpt_k_polar_express
    wb = L.gpt_k_polar_express_ws_bytes(12, 768, 768)
    assert wb > L.gpt_k_polar_express_ws_bytes(1, 768, 768) > 0
    assert L.gpt_k_polar_express_ws_bytes(1, 770, 768) == 0
    assert ns(A, 12, 770, 768, 1, A, 5, 1e-7, A, A, wb, None) == -1
    assert ns(A, 0, 768, 768, 1, A, 5, 1e-7, A, A, wb, None) == -1
    assert ns(A, 12, 768, 768, 1, None, 5, 1e-7, A, A, wb, None) == -1
    assert ns(A, 12, 768, 768, 1, A, 65, 1e-7, A, A, wb, None) == -1
    assert ns(A, 12, 768, 768, 1, A, 5, -1.0, A, A, wb, None) == -1
    assert ns(A, 12, 768, 768, 1, A, 5, 1e-7, A, A, wb - 1, None) == -3
    # optimizer elementwise steps
    assert L.gpt_k_muon_momentum(A, A, A, 6, 0.9, 1, 0, None) == -1
    assert L.gpt_k_muon_momentum(A, A, A, 8, 1.0, 1, 0, None) == -1
    assert L.gpt_k_muon_momentum(A, A, A, 8, 0.9, 1, 7, None) == -1
    assert L.gpt_k_muon_update(A, None, 8, 0.1, 0.0, None, None) == -1
    assert L.gpt_k_muon_update(A, A, 8, 0.1, 0.0, C.c_void_p(0x1004), None) == -4
    assert L.gpt_k_adamw(A, A, A, A, 8, 0, 1e-3, 0.9, 0.95, 1e-8, 0.0, None, None) == -1
    assert L.gpt_k_adamw(A, A, A, A, 8, 1, 1e-3, 1.5, 0.95, 1e-8, 0.0, None, None) == -1
    # optimizer step
    tc = G.make_config(gi.preset("tiny"))
    wsb = G.optim_ws_bytes(tc)
    hp = G.make_optim_hparams([(3.4445, -4.775, 2.0315)] * 5)
    assert wsb > 0
    assert L.gpt_optim_step(C.byref(tc), None, 1, A, None, A, A, A, A, wsb, None) == -1
    assert L.gpt_optim_step(C.byref(tc), C.byref(hp), 0, A, None, A, A, A, A, wsb, None) == -1
    assert L.gpt_optim_step(C.byref(tc), C.byref(hp), 1, A, None, A, A, A, A, wsb - 1, None) == -3
    bad_hp = G.make_optim_hparams([(3.4445, -4.775, 2.0315)] * 5, muon_momentum=1.0)
    assert L.gpt_optim_step(C.byref(tc), C.byref(bad_hp), 1, A, None, A, A, A, A, wsb, None) == -1
    bc = G.make_config(gi.preset("d4"))
    assert L.gpt_optim_step(C.byref(bc), C.byref(hp), 1, A, None, A, A, A, A,
                            G.optim_ws_bytes(bc), None) == -1      # bf16 needs params
    # model extras
    assert L.gpt_k_resid_mix_fwd(A, A, A, 12, A, 1, None) == -1
    assert L.gpt_k_resid_mix_fwd(A, A, A, 16, None, 1, None) == -1
    ms_ = L.gpt_k_resid_mix_bwd_scratch_bytes()
    assert L.gpt_k_resid_mix_bwd(A, A, A, None, A, 1, 16, A, A, A, ms_ - 1, 1, None) == -3
    assert L.gpt_k_resid_mix_bwd(A, A, A, None, A, 1, 16, A, None, A, ms_, 1, None) == -1
    assert L.gpt_k_smear_fwd(A, 2, 8, 20, A, A, C.c_void_p(0x2000), A, 1, None) == -1
    assert L.gpt_k_smear_fwd(A, 2, 8, 32, A, A, A, A, 1, None) == -1          # in place
    ss_ = L.gpt_k_smear_bwd_scratch_bytes()
    assert L.gpt_k_smear_bwd(A, C.c_void_p(0x2000), 2, 8, 32, A, A, A, C.c_void_p(0x3000), A,
                             A, ss_ - 1, 1, None) == -3
    # decode attention: q, kc, vc, lens, o, lse, B, Tq, Tmax, H, Hkv, hd, W, bound,
    # scratch, scratch_bytes, dtype
    dec = L.gpt_k_attn_decode
    nb = L.gpt_k_attn_decode_scratch_bytes(4, 1, 6, 2, 4096, 4096)
    assert nb > 0 and L.gpt_k_attn_decode_scratch_bytes(1, 1, 6, 4, 64, 64) == 0
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 128, 4096, 0.0, A, nb, 0, None) == -2
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 64, 4096, 0.0, A, nb, 1, None) == -2
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 4, 128, 4096, 0.0, A, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 100, 4096, 12, 1, 128, 4096, 0.0, A, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 1, 1 << 22, 6, 6, 128, 4096, 0.0, A, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 128, -1, 0.0, A, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 128, 4096, 64.0, A, nb, 1, None) == -1
    assert dec(A, A, A, None, A, A, 4, 1, 4096, 6, 2, 128, 4096, 0.0, A, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 128, 4096, 0.0, None, nb, 1, None) == -1
    assert dec(A, A, A, A, A, A, 4, 1, 4096, 6, 2, 128, 4096, 0.0, A, nb - 1, 1, None) == -3
    assert dec(A, A, A, A, C.c_void_p(0x1008), A, 4, 1, 4096, 6, 2, 128, 4096, 0.0, A, nb, 1,
               None) == -4


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert G.lib().gpt_status_string(s)
    assert G.lib().gpt_status_string(-99) == b"unknown status"


def test_no_cpu_fallback_in_product_path():
    """The binding and package never import the oracle."""
    pkg = os.path.join(ROOT, "gpt_pretraining_step_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f


def test_decode_noalloc_array_covers_every_decode_size():
    """The no-allocation decode entry's array holds the scratch of every
    size the regular decode entry accepts: the plan caps the split-key
    records (at most 510 chunk records), and a scan over batch, group
    width, query count and cache length never needs more than the cap."""
    cap = G.k_attn_decode_noalloc_max_scratch()
    worst = 0
    for B in (1, 2, 5, 17, 64, 85, 86, 128, 129, 255, 256, 1000):
        for Hkv in (1, 2, 3):
            for grp in (1, 3, 16, 33):
                for Tq in (1, 2, 16, 31):
                    if grp * Tq > 1024:
                        continue
                    for Tmax in (64, 4096, 100000):
                        for W in (0, 1024, Tmax):
                            worst = max(worst, G.k_attn_decode_scratch_bytes(
                                B, Tq, Hkv * grp, Hkv, Tmax, W))
    assert 0 < worst <= 4_244_224 <= cap
