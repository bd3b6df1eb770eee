"""End-to-end parity of gpt_step_fwd / gpt_step_bwd / gpt_eval_bpb against
the CPU oracle on identical seeded inputs (GPU only).

Bars: floating-point tensors within normwise max relative error 2e-2
(max|gpu - oracle| / max|oracle|) against the oracle's bf16-emulation mode
(fp32 mode for fp32 configs); val_bpb within 1e-3 absolute.
"""
import math
import sys

import numpy as np
import pytest

import gptinputs as gi
import oracle as O
from tests.gpu_util import grads_by_tensor, rel_err, small_bf16, tiny_plus, to_np, with_extras

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gpt_pretraining_step_amd as G  # noqa: E402
from gpt_pretraining_step_amd.session import Session  # noqa: E402

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _prec(cfg):
    return "bf16emu" if cfg["dtype"] == G.BF16 else "fp32"


def run_step(cfg, rows=None, accumulate_check=False):
    n = O.param_count(cfg)
    w, bits = with_extras(cfg, *gi.make_params(cfg, n))
    tok = gi.make_tokens(cfg, rows)
    if rows is not None:
        cfg = dict(cfg, batch=rows)
    s = Session(cfg)
    assert s.n_params == n
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    loss = float(s.loss.item())
    N = tok.shape[0] * (tok.shape[1] - 1)
    ell = to_np(s.ws_f32(G.WS_ELL, N))
    grads = to_np(s.grads)
    flag = int(s.ws[G.ws_offset(s.cfg, G.WS_NONFINITE):][:4].view(torch.int32).item())
    if accumulate_check:
        s.bwd(accumulate=True)
        torch.cuda.synchronize()
        g2 = to_np(s.grads)
        assert rel_err(g2, 2 * grads) < 1e-6
    return cfg, w, tok, loss, ell, grads, flag


def compare(cfg, w, tok, loss, ell, grads, flag):
    prec = _prec(cfg)
    ref_loss, ref_g, cache = O.step(cfg, w, tok, prec)
    assert flag == 0
    assert abs(loss - ref_loss) / abs(ref_loss) < (1e-3 if prec == "bf16emu" else 1e-5), \
        (loss, ref_loss)
    assert rel_err(ell, cache["ell"]) < TOL
    got = grads_by_tensor(cfg, grads)
    ref = grads_by_tensor(cfg, ref_g)
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    say("grad errors", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: (v, int(np.argmax(np.abs(got[k] - ref[k]))))
           for k, v in errs.items() if not v < (TOL if prec == "bf16emu" else 1e-4)}
    assert not bad, bad


@pytest.mark.parametrize("name", ["tiny", "tiny_plus", "small_bf16", "small_bf16_mha",
                                  "small_bf16_gqa_hd128", "small_bf16_wide_gate",
                                  "tiny_odd_gate", "d4", "tiny_T1", "small_bf16_T1"])
def test_step_matches_oracle(name):
    cfg = {"tiny": lambda: gi.preset("tiny"), "tiny_plus": tiny_plus,
           "small_bf16": small_bf16,
           "small_bf16_mha": lambda: small_bf16(n_kv_head=2, batch=2, seq_len=160,
                                                window_short=40, window_long=160,
                                                head_dim=128, n_head=2),
           # head dim 128 (the MFMA attention and its joint dK/dV pass) with two
           # query heads on one KV head and a ragged last 64-key block
           "small_bf16_gqa_hd128": lambda: small_bf16(n_kv_head=1, batch=2, seq_len=200,
                                                      window_short=72, window_long=200,
                                                      head_dim=128, n_head=2),
           # gate reading more channels than the fast gate-gradient path covers
           "small_bf16_wide_gate": lambda: small_bf16(ve_gate_channels=100),
           # a gate of 7 channels leaves later value-embedding tables off 16-byte
           # alignment: their gradients take the atomic scatter path
           "tiny_odd_gate": lambda: gi.preset("tiny", n_layer=4, window_pattern="SL",
                                              window_short=4, window_long=16, ve_every_odd=1,
                                              ve_gate_channels=7),
           "d4": lambda: gi.preset("d4"),
           # one-token rows (the degenerate sequence length)
           "tiny_T1": lambda: gi.preset("tiny", seq_len=1),
           "small_bf16_T1": lambda: small_bf16(seq_len=1, batch=5)}[name]()
    say("step", name)
    out = run_step(cfg, accumulate_check=(name == "tiny_plus"))
    compare(*out)


_EXTRAS = {
    # residual mixing, smear and backout after block 0 (bf16, GQA, windows,
    # value embeddings)
    "small_bf16_extras": lambda: small_bf16(resid_lambdas=1, smear=1, backout_layer=0),
    # smear and backout, no mixing, three layers (backing out the last
    # block's own output only rescales the stream the final RMSNorm sees, so
    # its lambda's gradient is a cancellation down to the norm's eps)
    "small_bf16_smear_backout": lambda: small_bf16(n_layer=3, smear=1, backout_layer=1),
    # mixing alone, four layers of fp32
    "tiny_resid_f32": lambda: gi.preset("tiny", n_layer=4, d_model=32, resid_lambdas=1),
    "tiny_extras_f32": lambda: dict(tiny_plus(), d_model=32, resid_lambdas=1, smear=1,
                                    backout_layer=1),
    "d4_extras": lambda: gi.preset("d4", resid_lambdas=1, smear=1, backout_layer=2),
    # one-token rows: every position starts its row (smear gates all zero,
    # attention sees only itself)
    "tiny_T1_extras_f32": lambda: dict(tiny_plus(), d_model=32, seq_len=1, resid_lambdas=1,
                                       smear=1, backout_layer=0),
    "small_bf16_T1_extras": lambda: small_bf16(seq_len=1, batch=5, resid_lambdas=1, smear=1,
                                               backout_layer=0),
}


@pytest.mark.parametrize("name", list(_EXTRAS))
def test_step_with_extras_matches_oracle(name):
    """The model extras inside the fused step (forward, backward, scalar
    gradients) against the oracle; gradient accumulation adds."""
    cfg = _EXTRAS[name]()
    say("step extras", name)
    out = run_step(cfg, accumulate_check=name in ("small_bf16_extras", "tiny_extras_f32"))
    compare(*out)


@pytest.mark.parametrize("name,n_rows", [("tiny", 11), ("small_bf16", 7), ("d4", 20),
                                         ("small_bf16_extras", 7)])
def test_eval_bpb_matches_oracle(name, n_rows):
    cfg = {"tiny": lambda: gi.preset("tiny"), "small_bf16": small_bf16,
           "d4": lambda: gi.preset("d4"), **_EXTRAS}[name]()
    say("eval", name, n_rows)
    n = O.param_count(cfg)
    w, bits = with_extras(cfg, *gi.make_params(cfg, n))
    tok = gi.make_eval_tokens(cfg, n_rows)          # ragged last batch
    tb = gi.make_token_bytes(cfg)
    s = Session(cfg, eval_ws=True, train_ws=False)
    s.set_params(w, bits)
    s.evaluate(s.upload(tok), s.upload(tb))
    torch.cuda.synchronize()
    got = s.bpb.cpu().numpy()
    nats, nbytes, bpb = O.eval_bpb(cfg, w, tok, tb, _prec(cfg))
    assert got[1] == nbytes
    assert abs(got[2] - bpb) < 1e-3, (got, bpb)
    assert abs(got[0] - nats) / nats < 1e-3


def _wlm_offset(cfg):
    off = 0
    for name, shape in O.param_layout(cfg):
        if name == "wlm":
            return off
        off += int(np.prod(shape))
    raise KeyError("wlm")


def test_step_far_apart_vocab_tiles():
    """lm_head rows of the first 256-entry vocabulary tile near +u and of the
    second near -u, |u| = 30: in about half the rows one tile's logits lie
    more than 40 below the other's, where the fused lm_head backward weighs
    the low tile at e^-40 instead of its (smaller) true weight.  Loss, losses
    and every gradient still match the oracle."""
    cfg = small_bf16(vocab=512)
    n = O.param_count(cfg)
    w, _ = with_extras(cfg, *gi.make_params(cfg, n))
    V, D = cfg["vocab"], cfg["d_model"]
    rng = np.random.default_rng(11)
    u = rng.standard_normal(D)
    u *= 30.0 / np.linalg.norm(u)
    wl = 0.02 * rng.standard_normal((V, D))
    wl[:256] += u
    wl[256:] -= u
    off = _wlm_offset(cfg)
    w = w.copy()
    w[off:off + V * D] = wl.reshape(-1)
    w, bits = with_extras(cfg, w, gi.bf16_bits_from_f32(w))
    tok = gi.make_tokens(cfg)
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    N = tok.shape[0] * (tok.shape[1] - 1)
    ell = to_np(s.ws_f32(G.WS_ELL, N))
    say("far-apart tiles: loss", float(s.loss.item()), "max loss", ell.max())
    assert ell.max() > 40.0          # some targets sit in the suppressed tile
    flag = int(s.ws[G.ws_offset(s.cfg, G.WS_NONFINITE):][:4].view(torch.int32).item())
    compare(cfg, w, tok, float(s.loss.item()), ell, to_np(s.grads), flag)


@pytest.mark.parametrize("vocab", [500, 512])
def test_uniform_logits_on_gpu(vocab):
    """With W_lm = 0 the loss is ln V exactly and every gradient but the
    lm_head's is exactly zero (closed form); V = 512 takes the fused
    lm_head / cross-entropy path, V = 500 the fp32-logits one."""
    cfg = small_bf16(vocab=vocab)
    n = O.param_count(cfg)
    w, bits = gi.make_params(cfg, n)
    off = O.param_count(cfg) - cfg["vocab"] * cfg["d_model"]
    w = w.copy(); bits = bits.copy()
    w[off:] = 0; bits[off:] = 0
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    s.fwd(); s.bwd()
    torch.cuda.synchronize()
    assert abs(s.loss.item() - math.log(cfg["vocab"])) < 1e-6
    g = to_np(s.grads)
    assert np.all(g[:off] == 0.0)
    assert np.abs(g[off:]).max() > 0


@pytest.mark.parametrize("vocab", [500, 512])
def test_nonfinite_flag(vocab):
    cfg = small_bf16(vocab=vocab)
    n = O.param_count(cfg)
    w, bits = gi.make_params(cfg, n)
    bits = bits.copy()
    bits[-5] = 0x7FC0                      # a NaN in W_lm
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    s.fwd()
    torch.cuda.synchronize()
    flag = int(s.ws[G.ws_offset(s.cfg, G.WS_NONFINITE):][:4].view(torch.int32).item())
    assert flag == 1
    assert not math.isfinite(s.loss.item())


def test_deterministic_forward():
    cfg = small_bf16()
    n = O.param_count(cfg)
    w, bits = gi.make_params(cfg, n)
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    s.fwd()
    torch.cuda.synchronize()
    N = cfg["batch"] * cfg["seq_len"]
    a = s.ws_f32(G.WS_ELL, N).clone()
    s.fwd()
    torch.cuda.synchronize()
    assert torch.equal(a, s.ws_f32(G.WS_ELL, N))


@pytest.mark.parametrize("extras", [False, True])
def test_deterministic_backward(extras):
    """Every gradient, the embedding tables' sorted scatter and the extras'
    scalar sums included, is a fixed-order sum: two backward passes agree
    bit for bit."""
    cfg = small_bf16(batch=4, seq_len=256)
    if extras:
        cfg.update(resid_lambdas=1, smear=1, backout_layer=0)
    n = O.param_count(cfg)
    w, bits = with_extras(cfg, *gi.make_params(cfg, n))
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    a = s.grads.clone()
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    assert torch.equal(a, s.grads)


def test_token_check():
    """With check_tokens on, in-range ids give the unchecked results bit
    for bit (the check only reads the tokens), and ids outside [0, V) make
    fwd, bwd and eval return GPT_ERR_INVALID_ARG before any gather runs
    (the loss buffer keeps its sentinel, the count sits in the workspace)."""
    cfg = small_bf16()
    n = O.param_count(cfg)
    w, bits = gi.make_params(cfg, n)
    tok = gi.make_tokens(cfg)
    ref = Session(cfg)
    ref.set_params(w, bits)
    ref.set_tokens(tok)
    ref.fwd()
    ref.bwd()
    s = Session(dict(cfg, check_tokens=1), eval_ws=True)
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    assert torch.equal(s.loss, ref.loss) and torch.equal(s.grads, ref.grads)
    V = cfg["vocab"]
    for bad_ids in ((-1,), (V,), (V, 2**31 - 1, -7)):
        say("token check", bad_ids)
        t = tok.copy()
        for i, b in enumerate(bad_ids):
            t[i % t.shape[0], 1 + 3 * i] = b
        s.set_tokens(t)
        s.loss.fill_(-123.0)
        with pytest.raises(G.GptError) as e:
            s.fwd()
        assert e.value.status == -1 and f"{len(bad_ids)} token ids" in str(e.value)
        with pytest.raises(G.GptError):
            s.bwd()
        with pytest.raises(G.GptError):
            s.evaluate(s.tokens, s.upload(gi.make_token_bytes(cfg)))
        torch.cuda.synchronize()
        assert s.loss.item() == -123.0
        off = G.ws_offset(s.cfg, G.WS_BAD_TOKENS)
        assert int(s.ws[off:off + 4].view(torch.int32).item()) == len(bad_ids)


@pytest.mark.parametrize("name", ["small", "small_extras", "d4"])
def test_two_stream_backward_equals_one_stream(name):
    """From 4096 tokens the backward runs its weight-gradient products and
    table gradients on a second stream (and, at head_dim 128, the attention
    dQ pass on a third).  Over two steps (the second accumulating), every
    gradient equals, bit for bit, the same backward on the caller's stream
    alone, except the linear layers' weight gradients: beside the main
    stream those products split K at most 4 ways (alone, as far as the plan
    likes), so they agree up to the fp32 summation order of the splits."""
    if name == "d4":
        cfg = gi.preset("d4")
    else:
        cfg = small_bf16(batch=16, seq_len=256)
    if name == "small_extras":
        cfg.update(resid_lambdas=1, smear=1, backout_layer=0)
    n = O.param_count(cfg)
    w, bits = with_extras(cfg, *gi.make_params(cfg, n))
    tok = gi.make_tokens(cfg)
    out = []
    for one in (0, 1):
        s = Session(dict(cfg, one_stream=one))
        s.set_params(w, bits)
        s.set_tokens(tok)
        s.fwd()
        s.bwd()
        s.fwd()
        s.bwd(accumulate=True)
        torch.cuda.synchronize()
        out.append(to_np(s.grads))
    a, b = grads_by_tensor(cfg, out[0]), grads_by_tensor(cfg, out[1])
    for k in a:
        if k.split(".")[-1] in ("wqkv", "wo", "wfc", "wproj"):
            assert rel_err(a[k], b[k]) < 1e-6, k
        else:
            assert np.array_equal(a[k], b[k]), k
