"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the oracle with a brute-force computation, a
closed form, an invariant, a library routine, or a value the pages print.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import gptinputs as gi
import oracle as O
from oracle.gpt import _Num
from tests.brute_force import brute_losses
from tests.gpu_util import set_extras

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_plus(**kw):
    """Tiny fixture with every feature on: 2 layers, 'SL' windows (S=4),
    value embeddings on layer 1 (gate over C=8 channels), G=2."""
    cfg = gi.preset("tiny", n_layer=2, window_pattern="SL", window_short=4,
                    window_long=16, ve_every_odd=1, ve_gate_channels=8)
    return cfg


def tiny_extras(**kw):
    """tiny_plus widened to D = 32 (smear reads 24 channels) with residual
    mixing, smear and backout after block 0 on."""
    return dict(tiny_plus(), **dict(dict(d_model=32, resid_lambdas=1, smear=1, backout_layer=0),
                                     **kw))


def inputs(cfg, rows=None, sigma=None):
    n = O.param_count(cfg)
    if sigma is not None:
        cfg = dict(cfg, sigma=sigma)
    w, _ = gi.make_params(cfg, n)
    return set_extras(cfg, w.astype(np.float64)), gi.make_tokens(cfg, rows)


# ---------------------------------------------------------------- P13, golden
def test_param_counts_closed_form():
    assert O.param_count(gi.preset("tiny")) == 3680
    # wte 432 + qkv 512 + o 256 + mlp 2048 + lm_head 432
    assert O.param_count(gi.preset("d12")) == 286_262_400
    assert O.param_count(gi.preset("d12gqa")) == 176_161_152
    assert O.param_count(gi.preset("d24")) == 1_384_124_928
    assert O.param_count(gi.preset("d4")) == 11_534_464


def test_microgpt_param_count_golden():
    """microgpt's printed ~4,192 parameters equal this layout (no biases, no
    norm gains, 4x MLP) at its shape once a learned position table is added
    and KV heads = query heads."""
    g = json.load(open(os.path.join(GOLDEN, "microgpt.json")))
    s = g["shape_reading"]
    cfg = gi.preset("tiny", n_kv_head=s["n_head"], n_head=s["n_head"],
                    head_dim=s["head_dim"], d_model=s["d_model"],
                    vocab=g["vocab"])
    assert O.param_count(cfg) + s["block_size"] * s["d_model"] == g["n_params"]


def test_init_loss_matches_microgpt_start():
    """P14: with N(0, sigma) lm_head on unit-RMS features, E[l] ~ ln V +
    sigma^2 D / 2; for the tiny model that is ~3.35, and microgpt prints a
    starting loss of ~3.3."""
    g = json.load(open(os.path.join(GOLDEN, "microgpt.json")))
    cfg = gi.preset("tiny", batch=64)
    w, tok = inputs(cfg)
    loss, _ = O.forward(cfg, w, tok, "fp64", keep=False)
    approx = math.log(27) + cfg["sigma"] ** 2 * cfg["d_model"] / 2
    assert abs(loss - approx) / approx < 0.03
    assert abs(loss - g["init_loss_approx"]) / g["init_loss_approx"] < g["init_loss_rel_tol"]


# ------------------------------------------------------------ brute force fwd
@pytest.mark.parametrize("which", ["tiny", "tiny_plus", "tiny_extras"])
def test_forward_equals_scalar_brute_force(which):
    cfg = {"tiny": lambda: gi.preset("tiny"), "tiny_plus": tiny_plus,
           "tiny_extras": tiny_extras}[which]()
    w, tok = inputs(cfg, rows=3)
    _, cache = O.forward(cfg, w, tok, "fp64", keep=False)
    ref = np.array(brute_losses(cfg, w, tok)).reshape(-1)
    np.testing.assert_allclose(cache["ell"], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------- P1 finite differences
def _fd_check(cfg, w, tok, coords):
    _, g, _ = O.step(cfg, w, tok, "fp64")
    eps = 1e-6
    fd = np.empty(len(coords))
    for n, i in enumerate(coords):
        wp = w.copy(); wp[i] += eps
        wm = w.copy(); wm[i] -= eps
        lp, _ = O.forward(cfg, wp, tok, "fp64", keep=False)
        lm, _ = O.forward(cfg, wm, tok, "fp64", keep=False)
        fd[n] = (lp - lm) / (2 * eps)
    an = g[coords]
    return np.linalg.norm(fd - an) / np.linalg.norm(an)


def test_finite_differences_tiny_all_params():
    cfg = gi.preset("tiny")
    w, tok = inputs(cfg)
    err = _fd_check(cfg, w, tok, np.arange(O.param_count(cfg)))
    assert err < 1e-6, err


@pytest.mark.parametrize("which", ["tiny_plus", "tiny_extras", "extras_no_resid"])
def test_finite_differences_tiny_plus_sampled(which):
    cfg = {"tiny_plus": tiny_plus, "tiny_extras": tiny_extras,
           "extras_no_resid": lambda: tiny_extras(resid_lambdas=0, backout_layer=1)}[which]()
    w, tok = inputs(cfg, rows=4)
    rng = np.random.default_rng(1)
    # a sample from every tensor, so no block's gradient goes unchecked
    coords, off = [], 0
    for _, shape in O.param_layout(cfg):
        n = int(np.prod(shape))
        coords += list(off + rng.choice(n, size=min(n, 120), replace=False))
        off += n
    err = _fd_check(cfg, w, tok, np.array(coords))
    assert err < 1e-6, err


def test_neutral_extras_equal_the_plain_model():
    """Mixing weights (1, 0), smear lambda 0 and backout lambda 0 leave the
    stream as it is: the loss and every shared gradient equal those of the
    same weights without the extras, and the extras' own gradients are the
    sums their definitions give (d lambda_r = sum dx . x_pre is nonzero)."""
    base = dict(tiny_plus(), d_model=32)
    cfg = tiny_extras()
    w, tok = inputs(base, rows=3)
    sl = O.extras_slots(cfg)
    ex = np.zeros(sl["size"])
    ex[0:2 * cfg["n_layer"]:2] = 1.0
    ex[sl["smear_w"]:sl["smear_w"] + 24] = 0.7
    l0, g0, _ = O.step(base, w, tok, "fp64")
    l1, g1, _ = O.step(cfg, np.concatenate([w, ex]), tok, "fp64")
    assert l1 == pytest.approx(l0, rel=1e-14)
    np.testing.assert_allclose(g1[:w.size], g0, rtol=1e-10, atol=1e-14)
    gex = g1[w.size:]
    assert np.all(gex[2 * cfg["n_layer"]:sl["smear_lambda"]] == 0.0)   # smear w: lambda 0
    assert abs(gex[0]) > 1e-6 and gex[sl["smear_lambda"]] != 0.0


def test_backout_of_the_last_block_only_rescales():
    """Backing out the last block's own output gives x (1 - lambda_b) ahead
    of the final RMSNorm: the loss equals the plain model's with the final
    stream scaled, and d loss / d lambda_b vanishes but for the norm's eps
    (here eps -> 1e-30 makes it exact to rounding)."""
    cfg = tiny_extras(resid_lambdas=0, smear=0, backout_layer=1, norm_eps=1e-30)
    w, tok = inputs(cfg, rows=3)
    sl = O.extras_slots(cfg)
    _, g, _ = O.step(cfg, w, tok, "fp64")
    assert abs(g[-sl["size"] + sl["backout"]]) < 1e-12
    base = dict(cfg, backout_layer=-1)
    l0, _ = O.forward(base, w[:-sl["size"]], tok, "fp64", keep=False)
    l1, _ = O.forward(cfg, w, tok, "fp64", keep=False)
    assert l1 == pytest.approx(l0, rel=1e-12)


# ------------------------------------------------------- P2 uniform logits
@pytest.mark.parametrize("name", ["tiny", "tiny_plus", "d4small"])
def test_uniform_logits_closed_form(name):
    if name == "tiny":
        cfg = gi.preset("tiny")
    elif name == "tiny_plus":
        cfg = tiny_plus()
    else:
        cfg = gi.preset("d4", n_layer=2, seq_len=32, batch=2, d_model=64,
                        n_head=2, n_kv_head=1, head_dim=32, vocab=300,
                        window_short=8, window_long=32, ve_gate_channels=16)
    w, tok = inputs(cfg)
    lay = O.param_layout(cfg)
    off = sum(int(np.prod(s)) for n, s in lay[:-1])
    w[off:] = 0.0                                        # W_lm = 0
    loss, g, cache = O.step(cfg, w, tok, "fp64")
    V = cfg["vocab"]
    assert loss == pytest.approx(math.log(V), abs=1e-12)
    # every gradient except dW_lm is exactly zero
    assert np.all(g[:off] == 0.0)
    B, T = tok.shape[0], tok.shape[1] - 1
    N = B * T
    hf = cache["hf"].reshape(N, -1)
    tgt = tok[:, 1:].reshape(-1)
    onehot = np.zeros((N, V)); onehot[np.arange(N), tgt] = 1
    ref = ((1.0 / V - onehot).T @ hf) / N
    np.testing.assert_allclose(g[off:].reshape(V, -1), ref, atol=1e-15)
    # bpb closed form
    tb = gi.make_token_bytes(cfg)
    nats, nbytes, bpb = O.eval_bpb(cfg, w, tok, tb, "fp64")
    assert nats == pytest.approx(N * math.log(V), rel=1e-13)
    assert bpb == pytest.approx(math.log(V) * N / (math.log(2) * tb[tgt].sum()), rel=1e-13)
    if name == "tiny":
        assert bpb == pytest.approx(math.log2(27), rel=1e-13)


# ------------------------------------------------------- attention invariants
def _rand_qkv(B=2, T=37, H=4, Hkv=2, hd=8, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, H, hd)), rng.standard_normal((B, T, Hkv, hd)),
            rng.standard_normal((B, T, Hkv, hd)))


@pytest.mark.parametrize("W", [0, 1, 5, 36, 100])
def test_attention_rows_stochastic_and_mask_exact(W):
    """P3/P4: probabilities of each query sum to 1; masked ones are 0.0."""
    q, k, v = _rand_qkv()
    num = _Num("fp64")
    _, lse = O.attention(q, k, v, W, num)
    for b in range(2):
        P, _, _ = O.gpt.attention_probs(q, k, lse, W, num, b)
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
        mask = O.visible_mask(q.shape[1], W)
        assert np.all(P[:, ~mask] == 0.0)
        assert np.all(P[:, mask] > 0.0)


def test_visible_mask_predicate():
    m = O.visible_mask(6, 2)
    for i in range(6):
        for j in range(6):
            assert m[i, j] == (j <= i and i - j <= 2)


@pytest.mark.parametrize("W", [0, 3, 17, 64])
def test_attention_matches_torch_sdpa(W):
    """Dense attention equals torch's scaled_dot_product_attention (CPU,
    float64) given the same boolean mask and KV heads repeated per group."""
    q, k, v = _rand_qkv(T=40)
    o, _ = O.attention(q, k, v, W, _Num("fp64"))
    G = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3)
    mask = torch.from_numpy(O.visible_mask(40, W))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_attention_bwd_matches_torch_autograd():
    q, k, v = _rand_qkv(T=29)
    W = 6
    num = _Num("fp64")
    o, lse = O.attention(q, k, v, W, num)
    do = np.random.default_rng(5).standard_normal(o.shape)
    dq, dk, dv = O.attention_bwd(q, k, v, o, lse, do, W, num)
    G = q.shape[2] // k.shape[2]
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    mask = torch.from_numpy(O.visible_mask(29, W))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.repeat_interleave(G, 2).permute(0, 2, 1, 3),
        tv.repeat_interleave(G, 2).permute(0, 2, 1, 3), attn_mask=mask)
    out.permute(0, 2, 1, 3).backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("W", [0, 127, 128, 200, 1000])
def test_dense_equals_tiled_online_softmax(W):
    """P16: the 128-key tiled online softmax (what the GPU runs) equals the
    dense definition."""
    q, k, v = _rand_qkv(B=1, T=300, H=2, Hkv=1, hd=16, seed=3)
    o, lse = O.attention(q, k, v, W, _Num("fp64"))
    ot, lset = O.attention_tiled(q, k, v, W)
    np.testing.assert_allclose(ot, o, atol=1e-12)
    np.testing.assert_allclose(lset, lse, atol=1e-12)


# ------------------------------------------------------- KV-cache decode
def _rand_cache(B=3, Tq=2, Tmax=23, H=4, Hkv=2, hd=8, seed=11):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Tq, H, hd)), rng.standard_normal((B, Tmax, Hkv, hd)),
            rng.standard_normal((B, Tmax, Hkv, hd)))


@pytest.mark.parametrize("W", [0, 2, 9, 100])
def test_decode_attention_matches_torch_sdpa(W):
    """Decode attention equals torch's scaled_dot_product_attention (CPU,
    float64) of each sequence's queries over its first L_b cache rows, with
    the boolean mask 0 <= p - j <= W written from the positions p = L_b - Tq
    + t; sequences of different lengths."""
    q, kc, vc = _rand_cache()
    lens = np.array([23, 9, 2])
    o, lse = O.decode_attention(q, kc, vc, lens, W, _Num("fp64"))
    B, Tq, H, hd = q.shape
    G = H // kc.shape[2]
    for b in range(B):
        L = int(lens[b])
        pos = np.arange(L - Tq, L)[:, None]
        j = np.arange(L)[None, :]
        mask = torch.from_numpy((pos - j >= 0) & (pos - j <= W))
        tq = torch.from_numpy(q[b]).permute(1, 0, 2)
        tk = torch.from_numpy(np.repeat(kc[b, :L], G, axis=1)).permute(1, 0, 2)
        tv = torch.from_numpy(np.repeat(vc[b, :L], G, axis=1)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        np.testing.assert_allclose(o[b], ref.permute(1, 0, 2).numpy(), atol=1e-12)
        s = np.einsum("thd,jhd->htj", q[b], np.repeat(kc[b, :L], G, axis=1)) / math.sqrt(hd)
        s = np.where(mask.numpy()[None], s, -np.inf)
        np.testing.assert_allclose(lse[b], np.log(np.exp(s).sum(-1)), atol=1e-12)


def test_decode_attention_is_the_last_rows_of_training_attention():
    """With the new tokens' keys in the cache, decode attention of the last Tq
    positions equals those rows of the dense causal attention over the whole
    sequence (the two masks are the same predicate)."""
    q_all, k, v = _rand_qkv(B=2, T=31, seed=7)
    for W in (0, 4, 30):
        o, lse = O.attention(q_all, k, v, W, _Num("fp64"))
        for Tq in (1, 3):
            od, lsed = O.decode_attention(q_all[:, -Tq:], k, v, np.array([31, 31]), W,
                                          _Num("fp64"))
            np.testing.assert_allclose(od, o[:, -Tq:], atol=1e-12)
            np.testing.assert_allclose(lsed, lse[:, :, -Tq:], atol=1e-12)


def test_decode_attention_closed_forms():
    """W = 0: the query sees only its own key, so o = v[p] and lse = q.k[p] /
    sqrt(hd).  Equal keys: o is the mean of the visible values and lse =
    score + log(count).  No visible key (L < Tq): o = 0, lse = -inf.  Rows at
    or past L never matter (NaN there changes nothing); lengths outside [0,
    Tmax] act as the nearest end."""
    q, kc, vc = _rand_cache(B=2, Tq=2, Tmax=12, H=2, Hkv=1, hd=4)
    num = _Num("fp64")
    lens = np.array([12, 5])
    o, lse = O.decode_attention(q, kc, vc, lens, 0, num)
    for b, L in enumerate(lens):
        for t in range(2):
            p = L - 2 + t
            for h in range(2):
                np.testing.assert_allclose(o[b, t, h], vc[b, p, 0], atol=1e-14)
                assert lse[b, h, t] == pytest.approx(q[b, t, h] @ kc[b, p, 0] / 2.0, abs=1e-14)
    kc_eq = np.broadcast_to(kc[:, :1], kc.shape).copy()
    o, lse = O.decode_attention(q, kc_eq, vc, lens, 3, num)
    for b, L in enumerate(lens):
        for t in range(2):
            p = L - 2 + t
            keys = [j for j in range(L) if 0 <= p - j <= 3]
            for h in range(2):
                np.testing.assert_allclose(o[b, t, h], vc[b, keys, 0].mean(0), atol=1e-14)
                sc = q[b, t, h] @ kc[b, 0, 0] / 2.0
                assert lse[b, h, t] == pytest.approx(sc + math.log(len(keys)), abs=1e-13)
    o, lse = O.decode_attention(q, kc, vc, np.array([1, 0]), 5, num)
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))
    assert np.all(o[0, 0] == 0.0) and np.all(np.isneginf(lse[0, :, 0]))
    np.testing.assert_allclose(o[0, 1, 0], vc[0, 0, 0], atol=1e-14)
    kn, vn = kc.copy(), vc.copy()
    kn[1, 5:], vn[1, 5:] = np.nan, np.nan
    a = O.decode_attention(q, kc, vc, lens, 7, num)
    bb = O.decode_attention(q, kn, vn, lens, 7, num)
    np.testing.assert_array_equal(a[0], bb[0])
    np.testing.assert_array_equal(a[1], bb[1])
    # lengths are clamped to [0, Tmax]
    hi = O.decode_attention(q, kc, vc, np.array([40, -3]), 7, num)
    ref = O.decode_attention(q, kc, vc, np.array([12, 0]), 7, num)
    np.testing.assert_array_equal(hi[0], ref[0])
    np.testing.assert_array_equal(hi[1], ref[1])


# ------------------------------------------------------- norm / rotary / CE
def test_rmsnorm_matches_torch():
    x = np.random.default_rng(0).standard_normal((5, 7, 24))
    y, r = O.rmsnorm(x, 1e-5, _Num("fp64"))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (24,), eps=1e-5)
    np.testing.assert_allclose(y, ref.numpy(), atol=1e-14)
    # P9: mean square after the norm is ms / (ms + eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-5), rtol=1e-13)


def test_rmsnorm_bwd_matches_torch_autograd():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 32)); dy = rng.standard_normal((6, 32))
    num = _Num("fp64")
    y, r = O.rmsnorm(x, 1e-5, num)
    tx = torch.tensor(x, requires_grad=True)
    torch.nn.functional.rms_norm(tx, (32,), eps=1e-5).backward(torch.from_numpy(dy))
    np.testing.assert_allclose(O.rmsnorm_bwd(dy, y, r, num), tx.grad.numpy(), atol=1e-13)


def test_rope_invariants():
    """P8: rotation preserves each pair's norm; q.k after rotation depends on
    positions only through their difference; rope then rms == rms then rope."""
    rng = np.random.default_rng(2)
    T, hd, s = 50, 16, 23
    num = _Num("fp64")
    x = rng.standard_normal((1, T, 3, hd))
    cos, sin = O.rope_tables(T + s, hd, 10000.0)
    y = O.rope(x, cos[:T], sin[:T], num)
    h = hd // 2
    np.testing.assert_allclose(x[..., :h] ** 2 + x[..., h:] ** 2,
                               y[..., :h] ** 2 + y[..., h:] ** 2, atol=1e-12)
    y2 = O.rope(x, cos[s:], sin[s:], num)            # every position + s
    d1 = np.einsum("bihd,bjhd->bhij", y, y)
    d2 = np.einsum("bihd,bjhd->bhij", y2, y2)
    np.testing.assert_allclose(d1, d2, atol=1e-11)
    a, _ = O.rmsnorm(O.rope(x, cos[:T], sin[:T], num), 1e-5, num)
    b = O.rope(O.rmsnorm(x, 1e-5, num)[0], cos[:T], sin[:T], num)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # rope_bwd is the inverse rotation
    np.testing.assert_allclose(O.rope_bwd(y, cos[:T], sin[:T], num), x, atol=1e-12)
    # half-split pairing and sign, written out for one pair (READING)
    t, j = 7, 3
    th = t * 10000.0 ** (-2 * j / hd)
    assert y[0, t, 0, j] == pytest.approx(x[0, t, 0, j] * math.cos(th) - x[0, t, 0, j + h] * math.sin(th))
    assert y[0, t, 0, j + h] == pytest.approx(x[0, t, 0, j] * math.sin(th) + x[0, t, 0, j + h] * math.cos(th))


def test_cross_entropy_matches_torch():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((33, 50)) * 3
    tgt = rng.integers(0, 50, 33)
    ell, lse, dz = O.cross_entropy(z, tgt, _Num("fp64"))
    tz = torch.tensor(z, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(tz, torch.from_numpy(tgt))
    loss.backward()
    assert ell.mean() == pytest.approx(loss.item(), abs=1e-13)
    np.testing.assert_allclose(dz, tz.grad.numpy(), atol=1e-15)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(z), 1).numpy(), atol=1e-13)


def test_round_bf16_matches_torch():
    x = np.random.default_rng(6).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.round_bf16(x), ref)


# ------------------------------------------------------- model-level invariants
def test_causal_prefix_invariance():
    """P6: changing tokens at positions >= t leaves losses at targets < t-1
    unchanged, bit for bit."""
    cfg = tiny_plus()
    w, tok = inputs(cfg, rows=2)
    t = 9
    tok2 = tok.copy()
    tok2[:, t:] = (tok2[:, t:] % 26) + 1
    for prec in ("fp64", "bf16emu"):
        _, c1 = O.forward(cfg, w, tok, prec, keep=False)
        _, c2 = O.forward(cfg, w, tok2, prec, keep=False)
        l1 = c1["ell"].reshape(2, -1)
        l2 = c2["ell"].reshape(2, -1)
        np.testing.assert_array_equal(l1[:, :t - 1], l2[:, :t - 1])
        assert np.any(l1[:, t - 1:] != l2[:, t - 1:])


def test_window_locality():
    """P7: in a one-layer model with window W, the loss at query i does not
    depend on the token at j < i - W."""
    cfg = gi.preset("tiny", window_pattern="S", window_short=3, window_long=16)
    w, tok = inputs(cfg, rows=1)
    j = 2
    tok2 = tok.copy(); tok2[0, j] = tok2[0, j] % 26 + 1
    _, c1 = O.forward(cfg, w, tok, "fp64", keep=False)
    _, c2 = O.forward(cfg, w, tok2, "fp64", keep=False)
    W = 3
    np.testing.assert_array_equal(c1["ell"][j + W + 1:], c2["ell"][j + W + 1:])
    assert c1["ell"][j + W] != c2["ell"][j + W]


def test_window_at_least_T_equals_full_causal():
    """P11."""
    cfg = gi.preset("tiny")
    w, tok = inputs(cfg)
    cfg_l = dict(cfg, window_pattern="L", window_long=cfg["seq_len"] + 5)
    _, c1 = O.forward(cfg, w, tok, "fp64", keep=False)
    _, c2 = O.forward(cfg_l, w, tok, "fp64", keep=False)
    np.testing.assert_array_equal(c1["ell"], c2["ell"])


def _to_mha(cfg, w):
    """Replicate GQA K/V weights, value-embedding columns and gate rows per
    group, giving an equivalent model with one KV head per query head."""
    H, Hkv, hd = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    G = H // Hkv
    P = O.unpack_params(cfg, w)
    mcfg = dict(cfg, n_kv_head=H)
    out = []
    for name, shape in O.param_layout(mcfg):
        t = P[name]
        if name.endswith("wqkv"):
            q = t[:H * hd]
            k = t[H * hd:(H + Hkv) * hd].reshape(Hkv, hd, -1)
            v = t[(H + Hkv) * hd:].reshape(Hkv, hd, -1)
            t = np.concatenate([q, np.repeat(k, G, 0).reshape(H * hd, -1),
                                np.repeat(v, G, 0).reshape(H * hd, -1)])
        elif name.endswith(".ve"):
            t = np.repeat(t.reshape(t.shape[0], Hkv, hd), G, 1).reshape(t.shape[0], -1)
        elif name.endswith(".wg"):
            t = np.repeat(t, G, 0)
        assert t.shape == shape
        out.append(t.reshape(-1))
    return mcfg, np.concatenate(out)


def test_gqa_equals_replicated_mha():
    """P10."""
    cfg = tiny_plus()
    w, tok = inputs(cfg, rows=2)
    mcfg, mw = _to_mha(cfg, w)
    l1, g1, _ = O.step(cfg, w, tok, "fp64")
    l2, g2, _ = O.step(mcfg, mw, tok, "fp64")
    assert l1 == pytest.approx(l2, abs=1e-12)
    # dW_k of the GQA model = sum over the group of the MHA model's dW_k
    H, Hkv, hd, D = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"], cfg["d_model"]
    G = H // Hkv
    G1 = O.unpack_params(cfg, g1)["l0.wqkv"]
    G2 = O.unpack_params(mcfg, g2)["l0.wqkv"]
    dk1 = G1[H * hd:(H + Hkv) * hd].reshape(Hkv, hd, D)
    dk2 = G2[H * hd:2 * H * hd].reshape(Hkv, G, hd, D).sum(1)
    np.testing.assert_allclose(dk1, dk2, atol=1e-12)


def test_value_embedding_special_cases():
    """P12: W_g = 0 gives gate 1.5 exactly; E_l = 0 gives the plain layer."""
    cfg = tiny_plus()
    w, tok = inputs(cfg, rows=2)
    P = O.unpack_params(cfg, w)
    P["l1.wg"][:] = 0.0
    _, c = O.forward(cfg, w, tok, "fp64")
    assert np.all(c["layers"][1]["g"] == 1.5)
    P["l1.ve"][:] = 0.0
    l1, _ = O.forward(cfg, w, tok, "fp64", keep=False)
    plain = dict(cfg, ve_every_odd=0)
    pw = np.concatenate([P[n].reshape(-1) for n, _ in O.param_layout(plain)])
    l2, _ = O.forward(plain, pw, tok, "fp64", keep=False)
    assert l1 == l2


def test_tiny_bpb_is_mean_loss_over_ln2():
    """P15: with every byte length 1, bpb = mean loss / ln 2."""
    cfg = gi.preset("tiny")
    w, tok = inputs(cfg)
    tb = gi.make_token_bytes(cfg)
    nats, nbytes, bpb = O.eval_bpb(cfg, w, tok, tb, "fp64")
    loss, _ = O.forward(cfg, w, tok, "fp64", keep=False)
    assert nbytes == tok[:, 1:].size
    assert bpb == pytest.approx(loss / math.log(2), rel=1e-14)


def test_eval_batches_are_additive():
    """Sums over a multi-batch set with a ragged last batch equal the sums
    of the batches taken one by one."""
    cfg = tiny_plus()
    w, _ = inputs(cfg)
    tok = gi.make_eval_tokens(cfg, 11)
    tb = gi.make_token_bytes(cfg)
    n1, b1, _ = O.eval_bpb(cfg, w, tok, tb, "fp64", rows_per_batch=4)
    n2 = sum(O.eval_bpb(cfg, w, tok[i:i + 1], tb, "fp64")[0] for i in range(11))
    assert n1 == pytest.approx(n2, rel=1e-13)


def test_bf16emu_close_to_fp32():
    """The rounding mode changes results only at bf16 level."""
    cfg = tiny_plus()
    w, tok = inputs(cfg, rows=4)
    l32, g32, _ = O.step(cfg, w.astype(np.float32), tok, "fp32")
    l16, g16, _ = O.step(cfg, w.astype(np.float32), tok, "bf16emu")
    assert abs(l32 - l16) < 1e-2
    assert np.abs(g32 - g16).max() / np.abs(g32).max() < 2e-2


# ------------------------------------------------------- FP8 (tensor-wise)
FP8 = ["e4m3", "e5m2"]
_TORCH_F8 = {"e4m3": "float8_e4m3fn", "e5m2": "float8_e5m2"}


@pytest.mark.parametrize("fmt", FP8)
def test_fp8_decode_matches_torch_and_encode_inverts_it(fmt):
    """All 256 codes: the field-definition decoder equals torch's view of the
    same bytes as its float8 dtype; encoding every finite value gives its
    code back."""
    from oracle import fp8
    codes = np.arange(256, dtype=np.uint8)
    v = fp8.fp8_decode(codes, fmt)
    ref = torch.from_numpy(codes.copy()).view(getattr(torch, _TORCH_F8[fmt])).double().numpy()
    np.testing.assert_array_equal(np.isnan(v), np.isnan(ref))
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(v[fin], ref[fin])
    np.testing.assert_array_equal(np.signbit(v[fin]), np.signbit(ref[fin]))
    np.testing.assert_array_equal(fp8.fp8_encode(v[fin], fmt), codes[fin])
    assert np.nanmax(v[np.isfinite(v)]) == fp8.FORMATS[fmt][3]


@pytest.mark.parametrize("fmt", FP8)
def test_fp8_round_is_nearest_even_by_brute_force(fmt):
    """Rounding equals a search over the sorted table of every finite value
    (nearest; a tie goes to the even code), on random values, every
    representable value and every midpoint; and equals torch's cast for the
    same in-range values."""
    from oracle import fp8
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.fp8_decode(codes, fmt)
    ok = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
    table, tcodes = vals[ok], codes[ok]
    order = np.argsort(table)
    table, tcodes = table[order], tcodes[order]
    fmax = fp8.FORMATS[fmt][3]
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-fmax, fmax, 4000),
                        rng.standard_normal(4000) * np.exp2(rng.integers(-20, 8, 4000)),
                        table, (table[1:] + table[:-1]) / 2])
    y = y[np.abs(y) <= fmax].astype(np.float32).astype(np.float64)
    got = fp8.fp8_round(y, fmt)
    d = np.abs(y[:, None] - table[None, :])
    best = d.min(1, keepdims=True)
    cand = d == best
    # among equally near values (a tie) take the even code
    even = (tcodes[None, :] & 1) == 0
    pick = np.where(cand.sum(1) > 1, np.argmax(cand & even, 1), np.argmax(cand, 1))
    np.testing.assert_array_equal(np.abs(got), np.abs(table[pick]))
    tt = torch.from_numpy(y).to(getattr(torch, _TORCH_F8[fmt])).double().numpy()
    np.testing.assert_array_equal(np.abs(got), np.abs(tt))


@pytest.mark.parametrize("fmt", FP8)
def test_fp8_quantize_scale(fmt):
    """The largest magnitude maps to +-fmax exactly; s = fmax / amax in fp32;
    an all-zero tensor gives zeros and s = fmax / 1e-12."""
    from oracle import fp8
    x = np.random.default_rng(5).standard_normal((7, 33)).astype(np.float32)
    x[3, 4] = -7.25
    codes, v, s, inv = fp8.quantize(x, fmt)
    fmax = fp8.FORMATS[fmt][3]
    assert s == np.float32(np.float32(fmax) / np.float32(7.25))
    assert v[3, 4] == -fmax and np.abs(v).max() == fmax
    assert inv == np.float32(1) / s
    np.testing.assert_array_equal(fp8.fp8_decode(codes, fmt), v)
    z = fp8.quantize(np.zeros((2, 16), np.float32), fmt)
    assert np.all(z[1] == 0) and z[2] == np.float32(np.float32(fmax) / np.float32(1e-12))
    # amax values where fp32(amax * s) lands above fmax: the clamp keeps the
    # largest element at fmax instead of overflowing the format
    amax = {"e4m3": np.float32(12.5159), "e5m2": np.float32(27.432611)}[fmt]
    s = np.float32(np.float32(fmax) / amax)
    assert np.float32(amax * s) > fmax
    _, v, _, _ = fp8.quantize(np.array([[amax, -amax / 3]], np.float32), fmt)
    assert v[0, 0] == fmax


def test_fp8_linear_exact_when_operands_are_representable():
    """x = k / 4 with |k| <= 14 and amax 3.5: s = 128 (a power of two), so
    every x s = 32 k is an e4m3 value and the FP8 product must equal the
    plain product exactly (rounded to bf16); the weight likewise with a
    different power of two.  A transposed operand or a wrong scale breaks
    this."""
    from oracle import fp8
    rng = np.random.default_rng(9)
    x = rng.integers(-14, 15, (37, 64)).astype(np.float32) / 4
    x[0, 0] = 3.5
    w = rng.integers(-12, 13, (21, 64)).astype(np.float32) / 32
    w[5, 7] = -448.0 / 1024           # amax 0.4375: s = 1024
    y = fp8.fp8_linear(x, w)
    ref = O.round_bf16((x.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32))
    np.testing.assert_array_equal(y, ref)
    _, qx, sx, ix = fp8.quantize(x, "e4m3")
    assert sx == 128 and ix == np.float32(1 / 128)
    np.testing.assert_array_equal(qx, x * 128)


# ------------------------------------------------------- Muon Newton-Schulz
PAGE_NS = [(8.156, -22.483, 15.879), (4.043, -2.809, 0.500)]


def test_polar_express_equals_the_matrix_quintic():
    """The oracle's SVD form equals the odd matrix quintic aX + bX(X^T X) +
    cX(X^T X)^2 evaluated directly with matrix products (fp64), one and two
    steps from X = G / ||G||_F, tall and wide; and on a diagonal matrix the
    result is the diagonal of the composed scalar quintic of d / ||d||
    (signs kept: the polynomials are odd)."""
    from oracle import muon
    rng = np.random.default_rng(0)
    for shape in ((40, 24), (24, 56)):
        G = rng.standard_normal(shape)
        for k in (1, 2):
            X = G / (np.linalg.norm(G) + muon.NS_EPS)
            for a, b, c in PAGE_NS[:k]:
                XtX = X.T @ X
                X = a * X + b * (X @ XtX) + c * (X @ XtX @ XtX)
            np.testing.assert_allclose(muon.polar_express(G, PAGE_NS[:k]), X, atol=1e-10)
    d = np.array([3.0, -1.0, 0.5, 2.0, -0.25])
    s = d / (np.linalg.norm(d) + muon.NS_EPS)
    for a, b, c in PAGE_NS:
        s = a * s + b * s ** 3 + c * s ** 5
    np.testing.assert_allclose(muon.polar_express(np.diag(d), PAGE_NS), np.diag(s), atol=1e-12)


def test_polar_express_orientation_scale_and_bf16():
    """A wide matrix is the transpose of its transpose's result; scaling G
    by a positive constant changes nothing but the eps term (the start
    divides by the norm);
    the bf16 mode stays within bf16 rounding of the exact iteration; the
    classic quintic Muon tuple iterated five times sends every singular
    value into a band around 1."""
    from oracle import muon
    rng = np.random.default_rng(1)
    G = rng.standard_normal((24, 56))
    X = muon.polar_express(G, PAGE_NS)
    np.testing.assert_allclose(X, muon.polar_express(G.T, PAGE_NS).T, atol=1e-12)
    np.testing.assert_allclose(muon.polar_express(7.5 * G, PAGE_NS), X, atol=1e-6)
    Xb = muon.polar_express(G, PAGE_NS, bf16=True)
    assert np.abs(Xb - X).max() / np.abs(X).max() < 3e-2
    classic = [(3.4445, -4.7750, 2.0315)] * 5
    sv = np.linalg.svd(muon.polar_express(rng.standard_normal((64, 32)), classic),
                       compute_uv=False)
    assert sv.min() > 0.6 and sv.max() < 1.25


def test_normuon_keeps_the_update_norm():
    """NorMuon only redistributes the update across neurons: the Frobenius
    norm of the scaled update equals the input's for any second-moment
    state; the state moves as v <- b2 v + (1 - b2) mean_c X^2 per row."""
    from oracle import muon
    rng = np.random.default_rng(3)
    for shape in ((48, 20), (16, 64)):
        X = rng.standard_normal(shape) * rng.uniform(0.1, 3.0, (shape[0], 1))
        v0 = rng.uniform(0.0, 2.0, shape[0])
        Y, v = muon.normuon(X, v0, 0.95)
        assert abs(np.linalg.norm(Y) - np.linalg.norm(X)) < 1e-12 * np.linalg.norm(X)
        np.testing.assert_allclose(v, 0.95 * v0 + 0.05 * (X ** 2).sum(1) / shape[1],
                                   rtol=1e-14)


def test_normuon_equalises_neurons_on_a_constant_series():
    """The same update t times from a zero state: the state is (1 - b2^t)
    times each row's mean square, and every row of the output has the same
    RMS, ||X||_F / sqrt(m n), whatever the rows' own scales (rows, not
    columns, are the neurons of an [out, in] weight)."""
    from oracle import muon
    rng = np.random.default_rng(4)
    m, n, b2 = 12, 40, 0.9
    X = rng.standard_normal((m, n)) * np.geomspace(0.01, 10.0, m)[:, None]
    v = np.zeros(m)
    for t in range(1, 6):
        Y, v = muon.normuon(X, v, b2)
        np.testing.assert_allclose(v, (1 - b2 ** t) * (X ** 2).mean(1), rtol=1e-12)
        row_rms = np.sqrt((Y ** 2).mean(1))
        np.testing.assert_allclose(row_rms, np.linalg.norm(X) / np.sqrt(m * n), rtol=1e-12)
        # each row keeps its direction
        np.testing.assert_allclose(Y / row_rms[:, None],
                                   X / np.sqrt((X ** 2).mean(1))[:, None], rtol=1e-12)


def test_normuon_special_cases():
    """Rows of equal RMS from a zero state come back unchanged (a +-1
    matrix); a zero row stays zero; an all-zero update gives zeros, not
    NaN (both norms clamp at 1e-10)."""
    from oracle import muon
    rng = np.random.default_rng(5)
    X = rng.choice([-1.0, 1.0], (8, 16))
    Y, _ = muon.normuon(X, np.zeros(8), 0.95)
    np.testing.assert_allclose(Y, X, rtol=1e-13)
    X[3] = 0.0
    X[5] *= 4.0
    Y, v = muon.normuon(X, np.zeros(8), 0.95)
    assert np.all(Y[3] == 0.0) and np.all(np.isfinite(Y)) and v[3] == 0.0
    Z, vz = muon.normuon(np.zeros((4, 8)), np.zeros(4), 0.95)
    assert np.all(Z == 0.0) and np.all(vz == 0.0)


def test_adamw_matches_torch():
    """Three AdamW steps equal torch.optim.AdamW (CPU, float64) on the same
    parameter and gradients, weights, moments and all."""
    from oracle import muon
    rng = np.random.default_rng(4)
    w0 = rng.standard_normal((6, 5))
    grads = [rng.standard_normal((6, 5)) for _ in range(3)]
    hp = dict(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-10, wd=0.1)
    p = torch.tensor(w0, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["wd"])
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    for k, g in enumerate(grads, 1):
        p.grad = torch.tensor(g)
        opt.step()
        w, m, v = muon.adamw(w, g, m, v, k, **hp)
    np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-15)
    st = opt.state[p]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_muon_momentum_and_update_closed_forms():
    """A constant gradient c gives momentum c (1 - beta^k) after k steps from
    zero, and the Nesterov update c (1 - beta^(k+1)); without Nesterov the
    update is the momentum.  The parameter step with no decay moves W by
    exactly -lr X; with decay it first scales W by 1 - lr wd."""
    from oracle import muon
    c = np.full((3, 4), 2.5)
    m = np.zeros_like(c)
    beta = 0.9
    for k in range(1, 6):
        m, u = muon.muon_momentum(c, m, beta)
        np.testing.assert_allclose(m, c * (1 - beta ** k), rtol=1e-14)
        np.testing.assert_allclose(u, c * (1 - beta ** (k + 1)), rtol=1e-14)
    m2, u2 = muon.muon_momentum(c, m, beta, nesterov=False)
    np.testing.assert_array_equal(u2, m2)
    w = np.arange(12.0).reshape(3, 4)
    x = np.ones((3, 4))
    np.testing.assert_allclose(muon.muon_update(w, x, 0.02, 0.0), w - 0.02, rtol=1e-15)
    np.testing.assert_allclose(muon.muon_update(w, x, 0.02, 0.5), w * 0.99 - 0.02, rtol=1e-15)


# ------------------------------------------------------- model extras
def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        g[i] = (f(xp) - f(xm)) / (2 * eps)
    return g


def test_extras_backward_by_finite_differences():
    """Every gradient of residual mixing, smear and backout equals central
    differences of a random linear functional of the output (fp64)."""
    from oracle import extras as X
    rng = np.random.default_rng(8)
    B, T, D = 2, 5, 28
    x, x0, xm = (rng.standard_normal((B * T, D)) for _ in range(3))
    c = rng.standard_normal((B * T, D))
    w = rng.standard_normal(24) * 0.3
    lr, l0, ls, lb = 0.9, 0.3, 0.7, 0.4
    dx, dx0, dlr, dl0 = X.resid_mix_bwd(c, x, x0, lr, l0)
    np.testing.assert_allclose(dx, _fd(lambda v: np.sum(c * X.resid_mix(v, x0, lr, l0)), x),
                               atol=1e-7)
    np.testing.assert_allclose(dx0, _fd(lambda v: np.sum(c * X.resid_mix(x, v, lr, l0)), x0),
                               atol=1e-7)
    assert dlr == pytest.approx(np.sum(c * x)) and dl0 == pytest.approx(np.sum(c * x0))
    sx, sw, sl = X.smear_bwd(c, x, w, ls, T)
    np.testing.assert_allclose(sx, _fd(lambda v: np.sum(c * X.smear(v, w, ls, T)[0]), x),
                               atol=1e-7)
    np.testing.assert_allclose(sw, _fd(lambda v: np.sum(c * X.smear(x, v, ls, T)[0]), w),
                               atol=1e-7)
    fl = _fd(lambda v: np.sum(c * X.smear(x, w, float(v[0]), T)[0]), np.array([ls]))
    assert sl == pytest.approx(fl[0], abs=1e-7)
    bx, bm, bl = X.backout_bwd(c, xm, lb)
    np.testing.assert_allclose(bm, _fd(lambda v: np.sum(c * X.backout(x, v, lb)), xm),
                               atol=1e-7)
    np.testing.assert_array_equal(bx, c)
    assert bl == pytest.approx(-np.sum(c * xm))


def test_extras_closed_forms():
    """lambda = 0 leaves the stream alone (smear, backout) or keeps only one
    input (mix); a zero gate weight gives g = lambda / 2, so y_t = x_t +
    (lambda / 2) x_(t-1) with the first position of every row untouched;
    backing out the stream itself with lambda 1 gives zero."""
    from oracle import extras as X
    rng = np.random.default_rng(9)
    T, D = 4, 30
    x, x0 = rng.standard_normal((2 * T, D)), rng.standard_normal((2 * T, D))
    np.testing.assert_array_equal(X.resid_mix(x, x0, 1.0, 0.0), x)
    np.testing.assert_array_equal(X.resid_mix(x, x0, 0.0, 1.0), x0)
    np.testing.assert_array_equal(X.smear(x, np.ones(24), 0.0, T)[0], x)
    y, g = X.smear(x, np.zeros(24), 0.8, T)
    for r in range(2):
        np.testing.assert_array_equal(y[r * T], x[r * T])
        for t in range(1, T):
            np.testing.assert_allclose(y[r * T + t], x[r * T + t] + 0.4 * x[r * T + t - 1],
                                       atol=1e-15)
    np.testing.assert_array_equal(X.backout(x, x, 1.0), np.zeros_like(x))
    np.testing.assert_array_equal(X.backout(x, x0, 0.0), x)


def test_batch_gradient_is_mean_of_row_gradients_in_the_oracle():
    """Rows never interact, so the oracle's gradient of a batch's mean loss
    equals the mean of its one-row gradients, and its evaluation sums are
    the sums of its rows' (fp64, tiny+ with windows, GQA and value
    embeddings) -- computed through the worker pool the full-size GPU tests
    use, so the pool's bookkeeping (row split, sums, order) is pinned too."""
    from tests.gpu_util import tiny_plus
    from tests import oracle_pool
    cfg = dict(tiny_plus(), batch=5)
    w, _ = gi.make_params(cfg, O.param_count(cfg))
    tok = gi.make_tokens(cfg)
    loss, g, _ = O.step(cfg, w, tok, "fp64")
    gm, losses = oracle_pool.mean_row_gradients(cfg, w, tok, "fp64", workers=2, cores=2)
    # the pool keeps fp32 partial sums
    assert np.abs(gm - g).max() <= 1e-6 * np.abs(g).max()
    assert abs(losses.mean() - loss) < 1e-12
    tb = gi.make_token_bytes(cfg)
    sums = oracle_pool.row_eval_sums(cfg, w, tok, tb, "fp64", workers=3, cores=3)
    ref = O.eval_bpb(cfg, w, tok, tb, "fp64")
    assert abs(sums[:, 0].sum() - ref[0]) < 1e-10 and sums[:, 1].sum() == ref[1]
