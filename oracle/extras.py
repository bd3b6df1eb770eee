"""Model extras found by the agent loop -- oracle (test infrastructure only).

[nanochat] "1. GPT model (nanochat/gpt.py)", efficiency tricks: per-layer
residual scaling x <- resid_lambda[i] x + x0_lambda[i] x0; smear, a gated mix
of the previous token's embedding (gate = smear_lambda sigmoid(smear_gate(
x[..., :24]))); backout, x <- x - backout_lambda x_backout with x_backout a
mid-layer residual.

READINGS (the page shows the three lines only):
  * x0 is the embedding output the blocks start from; the lambdas are
    scalar parameters, one pair per layer;
  * smear acts once on the embeddings: smear_gate is a bias-free linear map
    of the first 24 channels to one gate per token, x_pre_smear is the
    previous position's embedding in the same row (zero at the first
    position), so y_t = x_t + g_t x_(t-1);
  * backout acts once, after the last block: x_backout is the residual
    stream saved at a chosen middle layer.
Every function works on rows of tokens [N, D] in fp64 (exact), with a
backward that returns the gradients of every input.
"""
from __future__ import annotations

import numpy as np

SMEAR_CH = 24


def resid_mix(x, x0, lr: float, l0: float):
    return lr * np.asarray(x, np.float64) + l0 * np.asarray(x0, np.float64)


def resid_mix_bwd(dy, x, x0, lr: float, l0: float):
    """(dx, dx0, dlr, dl0)."""
    dy = np.asarray(dy, np.float64)
    return lr * dy, l0 * dy, float(np.sum(dy * x)), float(np.sum(dy * x0))


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def smear(x, w, lam: float, T: int):
    """x [N, D], N = B T; w [24]: y_t = x_t + g_t x_(t-1), g_t = lam
    sigmoid(w . x_t[:24]), no mix at the first position of each row."""
    x = np.asarray(x, np.float64)
    g = lam * _sig(x[:, :SMEAR_CH] @ np.asarray(w, np.float64))
    g = g.reshape(-1, T)
    g[:, 0] = 0.0
    g = g.reshape(-1)
    prev = np.zeros_like(x)
    xr, pr = x.reshape(-1, T, x.shape[1]), prev.reshape(-1, T, x.shape[1])
    pr[:, 1:] = xr[:, :-1]
    return x + g[:, None] * prev, g


def smear_bwd(dy, x, w, lam: float, T: int):
    """(dx, dw, dlam)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    w = np.asarray(w, np.float64)
    N, D = x.shape
    z = x[:, :SMEAR_CH] @ w
    s = _sig(z)
    first = (np.arange(N) % T) == 0
    g = np.where(first, 0.0, lam * s)
    prev = np.zeros_like(x)
    prev.reshape(-1, T, D)[:, 1:] = x.reshape(-1, T, D)[:, :-1]
    dg = np.where(first, 0.0, np.sum(dy * prev, axis=1))     # d y_t / d g_t
    dx = dy.copy()
    # the previous position receives g_t dy_t
    dxr = dx.reshape(-1, T, D)
    dxr[:, :-1] += (g[:, None] * dy).reshape(-1, T, D)[:, 1:]
    dz = dg * lam * s * (1.0 - s)
    dx[:, :SMEAR_CH] += dz[:, None] * w[None, :]
    dw = x[:, :SMEAR_CH].T @ dz
    dlam = float(np.sum(dg * s))
    return dx, dw, dlam


def backout(x, xm, lam: float):
    return np.asarray(x, np.float64) - lam * np.asarray(xm, np.float64)


def backout_bwd(dy, xm, lam: float):
    """(dx, dxm, dlam)."""
    dy = np.asarray(dy, np.float64)
    return dy, -lam * dy, float(-np.sum(dy * xm))
