"""Plain NumPy oracle of the GPT decoder step (test infrastructure only).

Precision modes
  'fp64'    : everything in float64, no rounding (finite differences, closed
              forms).
  'fp32'    : everything in float32, no rounding.
  'bf16emu' : float32 arithmetic, rounded to bf16 (nearest, ties to even) at
              exactly the points where the GPU path stores a bf16 tensor:
              embeddings, every normalised activation, qkv, v after the value
              embedding, q/k after rotary+QK-norm, attention output, the
              residual stream after each add (sum in fp32, rounded once), the
              MLP pre-activation u and activation a, dlogits, and every
              activation gradient at the same places.  Statistics (rstd, lse),
              logits, per-token losses and weight gradients stay fp32.

Model (one forward of the decoder; readings of the pages where they are silent
are marked READING):
  x  = wte[inp]                                     token embedding
  per layer l:
    h  = rms(x)                                     pre-norm, no gain (READING)
    q,k,v = split(h Wqkv^T)                         no biases (READING)
    if l odd: v += 3 sigmoid(h[:, :C] Wg^T) * E_l[inp]   [nanochat] value
                                                    embeddings, per-KV-head gate
    q,k = rms(rope(q)), rms(rope(k))                [nanochat] rotary + QK norm
    o  = softmax(q k^T / sqrt(hd) + mask_W) v       causal, window W_l, GQA
    x  = x + o Wo^T
    h2 = rms(x);  u = h2 Wfc^T;  a = relu(u)^2;  x = x + a Wproj^T
  hf = rms(x);  z = hf Wlm^T                        untied head
  loss = mean_n [ logsumexp(z_n) - z_n[tgt_n] ]     [microgpt] cross-entropy

Optional model extras ([nanochat] "1. GPT model", efficiency tricks; each
off unless the config turns it on; the arithmetic is in oracle/extras.py):
  smear=1          x = x + g x_prev right after the embedding, g = lambda_s
                   sigmoid(w_s . x[:24]) (zero at a row's first position)
  resid_lambdas=1  before block l: x = lr_l x + l0_l x0, x0 the stream the
                   blocks start from (after smear)
  backout_layer=j  the stream after block j is kept as x_mid; after the last
                   block x = x - lambda_b x_mid
The scalars and w_s live in one extra tensor "extras" after Wlm (READING: a
flat vector; its slots are listed at extras_slots).  In bf16emu every
extra's output is rounded once, like the residual adds.
"""
from __future__ import annotations

import math
import numpy as np

from . import extras as _ex

PRECISIONS = ("fp64", "fp32", "bf16emu")


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) \
        & np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(a.shape)


class _Num:
    """Working dtype and rounding hook for one precision mode."""

    def __init__(self, precision: str):
        if precision not in PRECISIONS:
            raise ValueError(precision)
        self.precision = precision
        self.dt = np.float64 if precision == "fp64" else np.float32

    def rnd(self, x):
        x = np.asarray(x, dtype=self.dt)
        return round_bf16(x) if self.precision == "bf16emu" else x


# --------------------------------------------------------------------------
# parameter layout: wte; per layer {Wqkv, Wo, Wfc, Wproj, [E_l, Wg]}; Wlm.
# every matrix is [out, in] row-major, as F.linear takes it ([nanochat]
# "3. precision management", the custom Linear).
# --------------------------------------------------------------------------
def is_ve_layer(cfg: dict, layer: int) -> bool:
    """Value embeddings on alternating layers; READING: 0-based odd layers."""
    return bool(cfg.get("ve_every_odd", 0)) and layer % 2 == 1


def extras_on(cfg: dict) -> bool:
    return bool(cfg.get("resid_lambdas", 0) or cfg.get("smear", 0)
                or cfg.get("backout_layer", -1) >= 0)


def extras_slots(cfg: dict) -> dict:
    """Slots of the "extras" vector: (lr_l, l0_l) at 2l, 2l+1; the smear
    weights w_s at 2L..2L+24, lambda_s at 2L+24, lambda_b at 2L+25; the
    length is padded to a multiple of 8."""
    L = cfg["n_layer"]
    return dict(smear_w=2 * L, smear_lambda=2 * L + 24, backout=2 * L + 25,
                size=8 * ((2 * L + 26 + 7) // 8))


def param_layout(cfg: dict):
    D, H, Hkv, hd = cfg["d_model"], cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    V, F, C = cfg["vocab"], cfg["mlp_mult"] * cfg["d_model"], cfg["ve_gate_channels"]
    out = [("wte", (V, D))]
    for l in range(cfg["n_layer"]):
        out += [(f"l{l}.wqkv", ((H + 2 * Hkv) * hd, D)),
                (f"l{l}.wo", (D, H * hd)),
                (f"l{l}.wfc", (F, D)),
                (f"l{l}.wproj", (D, F))]
        if is_ve_layer(cfg, l):
            out += [(f"l{l}.ve", (V, Hkv * hd)), (f"l{l}.wg", (Hkv, C))]
    out.append(("wlm", (V, D)))
    if extras_on(cfg):
        out.append(("extras", (extras_slots(cfg)["size"],)))
    return out


def param_count(cfg: dict) -> int:
    return int(sum(int(np.prod(s)) for _, s in param_layout(cfg)))


def unpack_params(cfg: dict, flat: np.ndarray) -> dict:
    flat = np.asarray(flat)
    if flat.size != param_count(cfg):
        raise ValueError("flat parameter size does not match the config")
    out, off = {}, 0
    for name, shape in param_layout(cfg):
        n = int(np.prod(shape))
        out[name] = flat[off:off + n].reshape(shape)
        off += n
    return out


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def rmsnorm(x, eps, num: _Num):
    """y = x / sqrt(mean(x^2) + eps) over the last axis, no gain.

    [microgpt] "model architecture": RMSNorm.  READING: no learnable gain
    (microgpt's ~4,192-parameter count leaves no room for one); eps added to
    the mean square inside the root.
    Returns (rounded y, r) with r = 1/sqrt(mean(x^2)+eps) unrounded.
    """
    x = np.asarray(x, dtype=num.dt)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + num.dt(eps))
    return num.rnd(x * r), r[..., 0].astype(num.dt)


def rmsnorm_bwd(dy, y, r, num: _Num):
    """Input gradient of y = x r(x):  dx = r (dy - y mean(dy*y)).

    Derivation: r = (mean x^2 + eps)^-1/2 so dr/dx_j = -r^3 x_j / D, hence
    dx_j = r dy_j - r^3 x_j sum_i(dy_i x_i)/D = r (dy_j - y_j mean(dy*y)).
    """
    dy = np.asarray(dy, dtype=num.dt)
    y = np.asarray(y, dtype=num.dt)
    m = np.mean(dy * y, axis=-1, keepdims=True)
    return (r[..., None] * (dy - y * m)).astype(num.dt)


def rope_tables(T: int, hd: int, base: float):
    """cos/sin [T, hd/2] in float64: theta_{t,j} = t * base^(-2j/hd).

    [nanochat] "1. GPT model": rotary embeddings, relative positions, no
    learned position table.  READING: the usual frequency ladder, base 10000,
    positions restart at 0 on every row.
    """
    j = np.arange(hd // 2, dtype=np.float64)
    inv = base ** (-2.0 * j / hd)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin, num: _Num):
    """Rotate pairs (j, j+hd/2) of x [B, T, heads, hd] by theta_{t,j}.

    READING: half-split pairing; y_j = x_j cos - x_{j+h} sin,
    y_{j+h} = x_j sin + x_{j+h} cos.
    """
    x = np.asarray(x, dtype=num.dt)
    h = x.shape[-1] // 2
    c = cos.astype(num.dt)[None, :, None, :]
    s = sin.astype(num.dt)[None, :, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(dy, cos, sin, num: _Num):
    """Gradient through rope(): the transpose rotation, i.e. angle -theta."""
    dy = np.asarray(dy, dtype=num.dt)
    h = dy.shape[-1] // 2
    c = cos.astype(num.dt)[None, :, None, :]
    s = sin.astype(num.dt)[None, :, None, :]
    d1, d2 = dy[..., :h], dy[..., h:]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def window_for_layer(cfg: dict, layer: int, T: int) -> int:
    """Attention window of a layer from the pattern string ([nanochat]
    "1. GPT model": sliding window with a pattern such as "SSSL").

    READING: character = pattern[layer mod len]; 'S' -> window_short,
    'L' -> window_long; an empty pattern means full causal (window T).
    """
    pat = cfg.get("window_pattern", "") or ""
    if not pat:
        return T
    ch = pat[layer % len(pat)]
    if ch == "S":
        return int(cfg["window_short"])
    if ch == "L":
        return int(cfg["window_long"])
    raise ValueError(f"bad window pattern character {ch!r}")


def visible_mask(T: int, W: int) -> np.ndarray:
    """mask[i, j] = key j visible from query i  <=>  0 <= i - j <= W.

    READING of the flash-attention call with causal=True and window_size
    ([nanochat] "5. flash attention integration"): the window counts keys to
    the left of the query, plus the query itself.
    """
    d = np.arange(T)[:, None] - np.arange(T)[None, :]
    return (d >= 0) & (d <= W)


def attention(q, k, v, W: int, num: _Num):
    """Dense causal/windowed grouped-query attention.

    q [B,T,H,hd], k/v [B,T,Hkv,hd].  Query head h reads KV head h // G,
    G = H / Hkv (READING: contiguous groups).  Scale 1/sqrt(hd).
    Returns o [B,T,H,hd] (rounded) and lse [B,H,T].
    """
    q = np.asarray(q, dtype=num.dt)
    B, T, H, hd = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    scale = num.dt(1.0 / math.sqrt(hd))
    mask = visible_mask(T, W)
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=num.dt)
    for b in range(B):
        qh = q[b].transpose(1, 0, 2)                                  # [H,T,hd]
        kh = np.repeat(np.asarray(k[b], num.dt).transpose(1, 0, 2), G, axis=0)
        vh = np.repeat(np.asarray(v[b], num.dt).transpose(1, 0, 2), G, axis=0)
        s = (qh @ kh.transpose(0, 2, 1)) * scale                      # [H,T,T]
        s = np.where(mask[None], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=-1, keepdims=True)
        lse[b] = (m + np.log(l))[..., 0]
        o[b] = ((p / l) @ vh).transpose(1, 0, 2)
    return num.rnd(o), lse


def attention_probs(q, k, lse, W: int, num: _Num, b: int):
    """P[h, i, j] of row b recomputed from q, k and the saved lse."""
    H, hd = q.shape[2], q.shape[3]
    G = H // k.shape[2]
    T = q.shape[1]
    scale = num.dt(1.0 / math.sqrt(hd))
    qh = np.asarray(q[b], num.dt).transpose(1, 0, 2)
    kh = np.repeat(np.asarray(k[b], num.dt).transpose(1, 0, 2), G, axis=0)
    s = (qh @ kh.transpose(0, 2, 1)) * scale
    p = np.exp(s - lse[b][..., None])
    return np.where(visible_mask(T, W)[None], p, num.dt(0)), qh, kh


def attention_bwd(q, k, v, o, lse, do, W: int, num: _Num):
    """Gradients of the attention above.

    Delta_i = sum_d dO_i o_i; dV = P^T dO; dP = dO V^T; dS = P (dP - Delta);
    dQ = dS K / sqrt(hd); dK = dS^T Q / sqrt(hd); dK, dV summed over the G
    query heads sharing a KV head.
    """
    B, T, H, hd = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    scale = num.dt(1.0 / math.sqrt(hd))
    dq = np.empty((B, T, H, hd), dtype=num.dt)
    dk = np.empty((B, T, Hkv, hd), dtype=num.dt)
    dv = np.empty((B, T, Hkv, hd), dtype=num.dt)
    for b in range(B):
        P, qh, kh = attention_probs(q, k, lse, W, num, b)
        vh = np.repeat(np.asarray(v[b], num.dt).transpose(1, 0, 2), G, axis=0)
        doh = np.asarray(do[b], num.dt).transpose(1, 0, 2)
        oh = np.asarray(o[b], num.dt).transpose(1, 0, 2)
        delta = np.sum(doh * oh, axis=-1, keepdims=True)
        dv_h = P.transpose(0, 2, 1) @ doh
        dP = doh @ vh.transpose(0, 2, 1)
        dS = P * (dP - delta)
        dq_h = (dS @ kh) * scale
        dk_h = (dS.transpose(0, 2, 1) @ qh) * scale
        dq[b] = dq_h.transpose(1, 0, 2)
        dk[b] = dk_h.reshape(Hkv, G, T, hd).sum(axis=1).transpose(1, 0, 2)
        dv[b] = dv_h.reshape(Hkv, G, T, hd).sum(axis=1).transpose(1, 0, 2)
    return num.rnd(dq), num.rnd(dk), num.rnd(dv)


def attention_tiled(q, k, v, W: int, tile: int = 128):
    """The same attention by 128-key tiles with an online (running max)
    softmax, in float64, skipping tiles that hold no visible key.  Used only
    to pin the tiled algebra against the dense definition."""
    q = np.asarray(q, np.float64)
    B, T, H, hd = q.shape
    G = H // k.shape[2]
    scale = 1.0 / math.sqrt(hd)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            kk = np.asarray(k[b, :, h // G], np.float64)
            vv = np.asarray(v[b, :, h // G], np.float64)
            for i0 in range(0, T, tile):
                qi = q[b, i0:i0 + tile, h]
                rows = np.arange(i0, min(T, i0 + tile))
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), hd))
                for j0 in range(0, T, tile):
                    cols = np.arange(j0, min(T, j0 + tile))
                    d = rows[:, None] - cols[None, :]
                    vis = (d >= 0) & (d <= W)
                    if not vis.any():
                        continue
                    s = np.where(vis, (qi @ kk[cols].T) * scale, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    # a row may see no key of this tile (and none before):
                    # its running max is still -inf and it gains nothing
                    dead = np.isinf(m_new)
                    m_safe = np.where(dead, 0.0, m_new)
                    alpha = np.where(np.isinf(m), 0.0, np.exp(m - m_safe))
                    p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
                    l = l * alpha + p.sum(axis=1)
                    acc = acc * alpha[:, None] + p @ vv[cols]
                    m = m_new
                o[b, rows, h] = acc / l[:, None]
                lse[b, h, rows] = m + np.log(l)
    return o, lse


def decode_attention(q, k_cache, v_cache, lens, W: int, num: _Num):
    """Attention of the newest tokens over a KV cache ([nanochat] "6.
    inference engine": prefilled caches, flash_attn_with_kvcache).

    q [B,Tq,H,hd]; k_cache/v_cache [B,Tmax,Hkv,hd]; lens[b] = L_b cached
    positions (clamped to [0, Tmax]).  READING: the Tq queries are the last
    Tq positions, p = L_b - Tq + t, and see key j < L_b iff 0 <= p - j <= W
    (the training mask); query head h reads KV head h // G; scale
    1/sqrt(hd).  Returns o [B,Tq,H,hd] (rounded) and lse [B,H,Tq]; a query
    that sees no key gets o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=num.dt)
    B, Tq, H, hd = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = H // Hkv
    scale = num.dt(1.0 / math.sqrt(hd))
    o = np.zeros_like(q)
    lse = np.full((B, H, Tq), -np.inf, dtype=num.dt)
    for b in range(B):
        L = min(max(int(lens[b]), 0), Tmax)
        for t in range(Tq):
            p = L - Tq + t
            j = np.arange(L)
            keys = j[(p - j >= 0) & (p - j <= W)]
            if len(keys) == 0:
                continue
            for h in range(H):
                kk = np.asarray(k_cache[b, keys, h // G], num.dt)
                vv = np.asarray(v_cache[b, keys, h // G], num.dt)
                sc = (kk @ q[b, t, h]) * scale
                m = sc.max()
                e = np.exp(sc - m)
                o[b, t, h] = (e / e.sum()) @ vv
                lse[b, h, t] = m + np.log(e.sum())
    return num.rnd(o), lse


def cross_entropy(z, tgt, num: _Num):
    """Per-token softmax cross-entropy on logits z [N, V].

    l_n = logsumexp(z_n) - z_n[tgt_n] (max-subtracted); dz = (softmax - onehot)/N
    for the mean over N tokens.  [microgpt] "training loop": cross-entropy of
    the next-token distribution.
    """
    z = np.asarray(z, dtype=num.dt)
    N = z.shape[0]
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    idx = np.arange(N)
    ell = lse - z[idx, tgt]
    p = np.exp(z - lse[:, None])
    p[idx, tgt] -= 1.0
    dz = p / num.dt(N)
    return ell.astype(num.dt), lse.astype(num.dt), dz.astype(num.dt)


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------
def _split_qkv(qkv, cfg):
    B, T, _ = qkv.shape
    H, Hkv, hd = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    q = qkv[..., :H * hd].reshape(B, T, H, hd)
    k = qkv[..., H * hd:(H + Hkv) * hd].reshape(B, T, Hkv, hd)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, T, Hkv, hd)
    return q, k, v


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def embedding(wte, inp, num: _Num):
    """x0 = wte[inp]: row lookup of the input ids ([microgpt] "model
    architecture": token embedding; [nanochat] "1. GPT model")."""
    return num.rnd(wte[inp])


def embedding_bwd(dx, inp, V: int):
    """dwte[v] = sum of dx over the positions whose input id is v (the
    transpose of the lookup)."""
    D = dx.shape[-1]
    dW = np.zeros((V, D), dtype=dx.dtype)
    np.add.at(dW, np.asarray(inp).reshape(-1), dx.reshape(-1, D))
    return dW


def value_embedding(v, h, wg, E, inp, C: int, num: _Num):
    """[nanochat] value-embedding snippet: per KV head, e = E[inp] and the
    gate g = 3 sigmoid(h[..., :C] wg^T) (READING: the first C channels of the
    normalised attention input); v + g e, rounded once.  Returns (v, g, e)."""
    B, T, Hkv, hd = v.shape
    e = E[inp].reshape(B, T, Hkv, hd)
    g = (3.0 * _sigmoid(h[..., :C] @ wg.T)).astype(num.dt)     # [B,T,Hkv]
    return num.rnd(v + g[..., None] * e), g, e


def value_embedding_bwd(dv, g, e, h, wg, inp, V: int):
    """Gradients of value_embedding from dv [B,T,Hkv,hd]: with s the sigmoid,
    dg = sum_d dv e, dzg = dg 3 s (1 - s) = dg g (1 - g/3); dwg = dzg^T h[:,
    :C]; dE[inp] += g dv; and the gate's share of dh[..., :C] is dzg wg.
    Returns (dzg, dwg, dE, dh_c)."""
    B, T, Hkv, hd = dv.shape
    C = wg.shape[1]
    dt = dv.dtype
    dgate = np.sum(dv * e, axis=-1)                             # [B,T,Hkv]
    dzg = dgate * g * (1.0 - g / 3.0)                           # 3s(1-s)
    dwg = (dzg.reshape(-1, Hkv).T @ h[..., :C].reshape(-1, C)).astype(dt)
    dE = np.zeros((V, Hkv * hd), dtype=dt)
    np.add.at(dE, np.asarray(inp).reshape(-1), (g[..., None] * dv).reshape(B * T, Hkv * hd))
    return dzg, dwg, dE, dzg @ wg


def forward(cfg: dict, flat_params, tokens, precision: str = "fp32",
            keep: bool = True):
    """One forward pass.  tokens [B, T+1] int; inputs are the first T ids,
    targets the last T (READING: rows of T+1 tokens).

    Returns (loss, cache).  cache['ell'] holds the per-token losses [B*T].
    """
    num = _Num(precision)
    dt = num.dt
    P = {k: np.asarray(v, dtype=dt) for k, v in unpack_params(cfg, flat_params).items()}
    tokens = np.asarray(tokens)
    B, T1 = tokens.shape
    T = T1 - 1
    inp, tgt = tokens[:, :T], tokens[:, 1:]
    H, Hkv, hd = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    C, eps = cfg["ve_gate_channels"], cfg["norm_eps"]
    cos, sin = rope_tables(T, hd, cfg["rope_base"])

    x = embedding(P["wte"], inp, num)                            # [B,T,D]
    D = x.shape[-1]
    ex = P.get("extras")
    sl = extras_slots(cfg)
    resid = bool(cfg.get("resid_lambdas", 0))
    bo = int(cfg.get("backout_layer", -1))
    if bo >= cfg["n_layer"] or (cfg.get("smear", 0) and D < _ex.SMEAR_CH):
        raise ValueError("backout_layer past the last block, or smear with d_model < 24")
    extra = {}
    if cfg.get("smear", 0):
        extra["x_emb"] = x
        y, _ = _ex.smear(x.reshape(-1, D), ex[sl["smear_w"]:sl["smear_w"] + _ex.SMEAR_CH],
                         ex[sl["smear_lambda"]], T)
        x = num.rnd(y.reshape(B, T, D))
    x0 = x
    layers = []
    for l in range(cfg["n_layer"]):
        c = {}
        if resid:
            c["x_pre"] = x
            x = num.rnd(_ex.resid_mix(x, x0, ex[2 * l], ex[2 * l + 1]))
        h, r = rmsnorm(x, eps, num)
        qkv = num.rnd(h @ P[f"l{l}.wqkv"].T)
        q, k, v = _split_qkv(qkv, cfg)
        if is_ve_layer(cfg, l):
            v, g, e = value_embedding(v, h, P[f"l{l}.wg"], P[f"l{l}.ve"], inp, C, num)
            c.update(e=e, g=g)
        q, rq = rmsnorm(rope(q, cos, sin, num), eps, num)
        k, rk = rmsnorm(rope(k, cos, sin, num), eps, num)
        W = window_for_layer(cfg, l, T)
        o, lse = attention(q, k, v, W, num)
        o2 = o.reshape(B, T, H * hd)
        x = num.rnd(x + o2 @ P[f"l{l}.wo"].T)
        h2, r2 = rmsnorm(x, eps, num)
        u = num.rnd(h2 @ P[f"l{l}.wfc"].T)
        a = num.rnd(np.maximum(u, 0) ** 2)
        x = num.rnd(x + a @ P[f"l{l}.wproj"].T)
        if l == bo:
            extra["x_mid"] = x
        if keep:
            c.update(h=h, r=r, q=q, k=k, v=v, rq=rq, rk=rk, o=o2, lse=lse,
                     W=W, h2=h2, r2=r2, u=u, a=a)
            layers.append(c)
    if bo >= 0:
        x = num.rnd(_ex.backout(x, extra["x_mid"], ex[sl["backout"]]))
    hf, rf = rmsnorm(x, eps, num)
    z = hf.reshape(B * T, -1) @ P["wlm"].T
    ell, lse_z, dz = cross_entropy(z, tgt.reshape(-1), num)
    loss = ell.astype(np.float64).mean()
    cache = dict(num=num, P=P, inp=inp, tgt=tgt, B=B, T=T, cos=cos, sin=sin,
                 ell=ell, lse_z=lse_z, loss=loss)
    if keep:
        cache.update(layers=layers, hf=hf, rf=rf, dz=num.rnd(dz), z=z, x0=x0, **extra)
    return loss, cache


def backward(cfg: dict, cache: dict) -> dict:
    """Explicit reverse-mode gradients of the mean loss, one step at a time
    (the style of microgpt's explicit-backprop variants).  Returns fp32/fp64
    gradients keyed like param_layout."""
    num = cache["num"]
    dt = num.dt
    P, inp = cache["P"], cache["inp"]
    B, T = cache["B"], cache["T"]
    H, Hkv, hd = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    C, D = cfg["ve_gate_channels"], cfg["d_model"]
    cos, sin = cache["cos"], cache["sin"]
    grads = {}

    dz = cache["dz"]                                             # [N,V]
    hf = cache["hf"].reshape(B * T, D)
    grads["wlm"] = (dz.T @ hf).astype(dt)
    dhf = num.rnd(dz @ P["wlm"]).reshape(B, T, D)
    dx = num.rnd(rmsnorm_bwd(dhf, cache["hf"], cache["rf"], num))
    ex = P.get("extras")
    sl = extras_slots(cfg)
    resid = bool(cfg.get("resid_lambdas", 0))
    bo = int(cfg.get("backout_layer", -1))
    if ex is not None:
        gex = np.zeros(ex.shape, dtype=np.float64)
    if bo >= 0:
        # x_out = x - lambda_b x_mid: dx passes through, x_mid gets -lambda_b dx
        _, dxm, gex[sl["backout"]] = _ex.backout_bwd(dx, cache["x_mid"], ex[sl["backout"]])
        dxm = num.rnd(dxm)
    dx0 = None

    for l in reversed(range(cfg["n_layer"])):
        c = cache["layers"][l]
        if l == bo:
            dx = num.rnd(dx + dxm)
        # MLP: x_out = x_mid + a Wproj^T,  a = relu(u)^2,  u = h2 Wfc^T
        grads[f"l{l}.wproj"] = (dx.reshape(-1, D).T
                                @ c["a"].reshape(B * T, -1)).astype(dt)
        da = dx @ P[f"l{l}.wproj"]
        du = num.rnd(da * (2.0 * np.maximum(c["u"], 0)))
        grads[f"l{l}.wfc"] = (du.reshape(B * T, -1).T
                              @ c["h2"].reshape(B * T, D)).astype(dt)
        dh2 = num.rnd(du @ P[f"l{l}.wfc"])
        dx = num.rnd(dx + rmsnorm_bwd(dh2, c["h2"], c["r2"], num))
        # attention: x_mid = x_in + o Wo^T
        grads[f"l{l}.wo"] = (dx.reshape(-1, D).T
                             @ c["o"].reshape(B * T, -1)).astype(dt)
        do = num.rnd(dx @ P[f"l{l}.wo"]).reshape(B, T, H, hd)
        dq, dk, dv = attention_bwd(c["q"], c["k"], c["v"],
                                   c["o"].reshape(B, T, H, hd), c["lse"], do,
                                   c["W"], num)
        # QK-norm then rotary, backwards
        dq = num.rnd(rope_bwd(rmsnorm_bwd(dq, c["q"], c["rq"], num), cos, sin, num))
        dk = num.rnd(rope_bwd(rmsnorm_bwd(dk, c["k"], c["rk"], num), cos, sin, num))
        dqkv = np.concatenate([dq.reshape(B, T, -1), dk.reshape(B, T, -1),
                               dv.reshape(B, T, -1)], axis=-1)
        dh = num.rnd(dqkv @ P[f"l{l}.wqkv"])
        grads[f"l{l}.wqkv"] = (dqkv.reshape(B * T, -1).T
                               @ c["h"].reshape(B * T, D)).astype(dt)
        if is_ve_layer(cfg, l):
            # v = v_lin + g * e,  g = 3 sigmoid(zg),  zg = h[:, :C] Wg^T
            _, dwg, dE, dh_c = value_embedding_bwd(dv.astype(dt), c["g"], c["e"], c["h"],
                                                   P[f"l{l}.wg"], inp, P[f"l{l}.ve"].shape[0])
            grads[f"l{l}.wg"] = dwg
            grads[f"l{l}.ve"] = dE
            dh = dh.astype(dt).copy()
            dh[..., :C] += dh_c
        dx = num.rnd(dx + rmsnorm_bwd(dh, c["h"], c["r"], num))
        if resid:
            # x = lr x_pre + l0 x0: x0's gradient gathers over the layers
            dxp, dx0l, gex[2 * l], gex[2 * l + 1] = _ex.resid_mix_bwd(
                dx, c["x_pre"], cache["x0"], ex[2 * l], ex[2 * l + 1])
            dx0 = num.rnd(dx0l if dx0 is None else dx0 + dx0l)
            dx = num.rnd(dxp)

    if resid:
        dx = num.rnd(dx + dx0)
    if cfg.get("smear", 0):
        D = dx.shape[-1]
        w = ex[sl["smear_w"]:sl["smear_w"] + _ex.SMEAR_CH]
        dxe, dw, dlam = _ex.smear_bwd(dx.reshape(-1, D), cache["x_emb"].reshape(-1, D), w,
                                      ex[sl["smear_lambda"]], T)
        gex[sl["smear_w"]:sl["smear_w"] + _ex.SMEAR_CH] = dw
        gex[sl["smear_lambda"]] = dlam
        dx = num.rnd(dxe).reshape(B, T, D)
    grads["wte"] = embedding_bwd(dx, inp, P["wte"].shape[0])
    if ex is not None:
        grads["extras"] = gex.astype(dt)
    return grads


def flatten_grads(cfg: dict, grads: dict) -> np.ndarray:
    return np.concatenate([np.asarray(grads[n]).reshape(-1)
                           for n, _ in param_layout(cfg)])


def step(cfg: dict, flat_params, tokens, precision: str = "fp32"):
    """Forward + backward: returns (loss, flat gradients, cache)."""
    loss, cache = forward(cfg, flat_params, tokens, precision)
    return loss, flatten_grads(cfg, backward(cfg, cache)), cache


def eval_bpb(cfg: dict, flat_params, tokens, token_bytes, precision="fp32",
             rows_per_batch: int | None = None):
    """Bits per byte over every row of an evaluation set.

    bpb = sum_n l_n / (ln 2 * sum_n bytes[tgt_n]) ([autoresearch] "core
    mechanism": validation bits per byte, vocabulary-independent).  Rows are
    processed in batches of the config's batch size; sums are float64.
    Returns (sum_nats, sum_bytes, bpb).
    """
    tokens = np.asarray(tokens)
    tb = np.asarray(token_bytes, dtype=np.int64)
    Bsz = rows_per_batch or cfg["batch"]
    nats, nbytes = 0.0, 0
    for r0 in range(0, tokens.shape[0], Bsz):
        rows = tokens[r0:r0 + Bsz]
        _, cache = forward(cfg, flat_params, rows, precision, keep=False)
        nats += float(np.sum(cache["ell"].astype(np.float64)))
        nbytes += int(np.sum(tb[rows[:, 1:]]))
    return nats, float(nbytes), nats / (math.log(2.0) * nbytes)
