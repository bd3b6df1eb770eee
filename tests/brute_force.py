"""Scalar pure-Python forward of the decoder, for tiny inputs only.

Written independently of the vectorised oracle (own parameter walk, explicit
loops over tokens, heads and channels, Python floats = IEEE double) so that
an index, sign or transpose slip in either one shows up as a mismatch.  It
follows the same readings: pre-norm RMSNorm without gain, half-split rotary
pairs with theta = t * base^(-2j/hd), QK-norm after rotary, key j visible from
query i iff 0 <= i-j <= W, KV head of query head h is h // (H/Hkv), value
embeddings with gate 3*sigmoid(.) on odd layers, ReLU^2 MLP, untied head;
and, when the config turns them on, the model extras: smear of the previous
position's embedding right after the lookup, per-block mixing with the
post-smear stream before every block, and backout of the stream after block
`backout_layer` once all blocks ran.  The extras vector follows Wlm: pairs
(resid, x0) per layer, 24 smear weights, smear lambda, backout lambda.
"""
import math


def _take(flat, off, rows, cols):
    m = [[float(flat[off + r * cols + c]) for c in range(cols)] for r in range(rows)]
    return m, off + rows * cols


def _matvec(W, x):
    return [sum(wr[i] * x[i] for i in range(len(x))) for wr in W]


def _rms(x, eps):
    r = 1.0 / math.sqrt(sum(v * v for v in x) / len(x) + eps)
    return [v * r for v in x]


def brute_losses(cfg, flat, tokens):
    """Per-token losses [B][T] of the forward pass, pure Python."""
    D, H, Hkv, hd = cfg["d_model"], cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    V, L, C = cfg["vocab"], cfg["n_layer"], cfg["ve_gate_channels"]
    F = cfg["mlp_mult"] * D
    eps, base = cfg["norm_eps"], cfg["rope_base"]
    G = H // Hkv
    off = 0
    wte, off = _take(flat, off, V, D)
    layers = []
    for l in range(L):
        p = {}
        p["wqkv"], off = _take(flat, off, (H + 2 * Hkv) * hd, D)
        p["wo"], off = _take(flat, off, D, H * hd)
        p["wfc"], off = _take(flat, off, F, D)
        p["wproj"], off = _take(flat, off, D, F)
        if cfg.get("ve_every_odd") and l % 2 == 1:
            p["ve"], off = _take(flat, off, V, Hkv * hd)
            p["wg"], off = _take(flat, off, Hkv, C)
        pat = cfg.get("window_pattern") or ""
        if not pat:
            p["W"] = 10 ** 9
        else:
            ch = pat[l % len(pat)]
            p["W"] = cfg["window_short"] if ch == "S" else cfg["window_long"]
        layers.append(p)
    wlm, off = _take(flat, off, V, D)
    resid = bool(cfg.get("resid_lambdas", 0))
    smear = bool(cfg.get("smear", 0))
    bo = int(cfg.get("backout_layer", -1))
    if resid or smear or bo >= 0:
        n_ex = 8 * ((2 * L + 26 + 7) // 8)
        ex = [float(v) for v in flat[off:off + n_ex]]
        off += n_ex
    assert off == len(flat)

    out = []
    for row in tokens:
        row = [int(t) for t in row]
        T = len(row) - 1
        xs = [list(wte[row[t]]) for t in range(T)]
        if smear:
            ws, lam = ex[2 * L:2 * L + 24], ex[2 * L + 24]
            emb = [list(x) for x in xs]
            for t in range(1, T):
                z = sum(ws[c] * emb[t][c] for c in range(24))
                gate = lam / (1.0 + math.exp(-z))
                xs[t] = [emb[t][d] + gate * emb[t - 1][d] for d in range(D)]
        x0s = [list(x) for x in xs]
        for li, p in enumerate(layers):
            if resid:
                xs = [[ex[2 * li] * xs[t][d] + ex[2 * li + 1] * x0s[t][d] for d in range(D)]
                      for t in range(T)]
            hs = [_rms(x, eps) for x in xs]
            qs, ks, vs = [], [], []
            for t in range(T):
                qkv = _matvec(p["wqkv"], hs[t])
                q = [qkv[h * hd:(h + 1) * hd] for h in range(H)]
                k = [qkv[(H + g) * hd:(H + g + 1) * hd] for g in range(Hkv)]
                v = [qkv[(H + Hkv + g) * hd:(H + Hkv + g + 1) * hd] for g in range(Hkv)]
                if "ve" in p:
                    e = p["ve"][row[t]]
                    for g in range(Hkv):
                        zg = sum(p["wg"][g][c] * hs[t][c] for c in range(C))
                        gate = 3.0 / (1.0 + math.exp(-zg))
                        v[g] = [v[g][d] + gate * e[g * hd + d] for d in range(hd)]

                def rot(vec):
                    half = hd // 2
                    o = [0.0] * hd
                    for j in range(half):
                        th = t * base ** (-2.0 * j / hd)
                        a, b = vec[j], vec[j + half]
                        o[j] = a * math.cos(th) - b * math.sin(th)
                        o[j + half] = a * math.sin(th) + b * math.cos(th)
                    return _rms(o, eps)

                qs.append([rot(x) for x in q])
                ks.append([rot(x) for x in k])
                vs.append(v)
            new_x = []
            for i in range(T):
                o_cat = []
                for h in range(H):
                    g = h // G
                    js = [j for j in range(T) if 0 <= i - j <= p["W"]]
                    s = [sum(qs[i][h][d] * ks[j][g][d] for d in range(hd)) / math.sqrt(hd)
                         for j in js]
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    tot = sum(w)
                    o_cat += [sum(w[n] * vs[js[n]][g][d] for n in range(len(js))) / tot
                              for d in range(hd)]
                x = [xs[i][d] + y for d, y in enumerate(_matvec(p["wo"], o_cat))]
                h2 = _rms(x, eps)
                a = [max(u, 0.0) ** 2 for u in _matvec(p["wfc"], h2)]
                x = [x[d] + y for d, y in enumerate(_matvec(p["wproj"], a))]
                new_x.append(x)
            xs = new_x
            if li == bo:
                mid = [list(x) for x in xs]
        if bo >= 0:
            xs = [[xs[t][d] - ex[2 * L + 25] * mid[t][d] for d in range(D)] for t in range(T)]
        losses = []
        for t in range(T):
            z = _matvec(wlm, _rms(xs[t], eps))
            m = max(z)
            lse = m + math.log(sum(math.exp(v - m) for v in z))
            losses.append(lse - z[row[t + 1]])
        out.append(losses)
    return out
