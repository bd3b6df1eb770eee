"""Muon and AdamW optimizer steps -- oracle (test infrastructure only).

[nanochat] "2. Muon optimizer (nanochat/optim.py)": the update of a matrix
parameter is orthogonalized by a quintic Newton-Schulz iteration ("Polar
Express"): per coefficient tuple (a, b, c), A = X^T X, B = b A + c A A,
X <- a X + X B.  The page prints the first two of five tuples and elides
the rest, so the tuples are an input here.

READINGS (the page shows the loop only):
  * start: X = G / (||G||_F + eps), eps = 1e-7 (the iteration is built for
    singular values at most 1; Muon's normalisation);
  * orientation: the loop as printed (Gram matrix X^T X) for a matrix with
    at least as many rows as columns; a wider matrix is iterated as its
    transpose, so the Gram matrix is always the smaller side;
  * precision: X, A and B are bf16 between the products (Muon runs the
    iteration in bf16); products accumulate exactly here.
"""
from __future__ import annotations

import numpy as np

from .gpt import round_bf16

NS_EPS = 1e-7


def _rnd(x, bf16: bool):
    return round_bf16(np.asarray(x, np.float32)).astype(np.float64) if bf16 else x


def polar_express(G, coeffs, eps: float = NS_EPS, bf16: bool = False) -> np.ndarray:
    """The orthogonalized update of G [m, n] (fp64, or with bf16 storage of
    X, A and B when bf16 is set)."""
    G = np.asarray(G, np.float64)
    if G.shape[0] < G.shape[1]:
        return polar_express(G.T, coeffs, eps, bf16).T
    X = _rnd(G / (np.linalg.norm(G) + eps), bf16)
    for a, b, c in coeffs:
        A = _rnd(X.T @ X, bf16)
        B = _rnd(b * A + c * (A @ A), bf16)
        X = _rnd(a * X + X @ B, bf16)
    return X


def ns_flops(m: int, n: int, steps: int) -> float:
    """Multiply-add flops of the iteration: per step X^T X (2 m n^2), A A
    (2 n^3) and X B (2 m n^2), with n the smaller side."""
    m, n = max(m, n), min(m, n)
    return steps * (4.0 * m * n * n + 2.0 * n ** 3)


# --------------------------------------------------------------------------
# the elementwise parts of the optimizer step
# --------------------------------------------------------------------------
# READINGS: the page names Muon (momentum, orthogonalized update) for the
# block matrices and AdamW for embeddings, lm_head and value embeddings, and
# prints neither the momentum form nor the AdamW constants, so the published
# definitions are used with every constant an argument: Muon's momentum
# buffer M <- beta M + (1 - beta) G with the Nesterov look-ahead
# (1 - beta) G + beta M as the update fed to the orthogonalization; the
# parameter step W <- W (1 - lr wd) - lr X (decoupled decay, lr carrying any
# shape factor); AdamW as Loshchilov & Hutter with bias correction.  The
# NorMuon rescaling is not modelled: its snippet uses symbols the page never
# defines.

def muon_momentum(grad, mom, beta: float, nesterov: bool = True):
    """(new momentum, the update to orthogonalize), fp64."""
    grad = np.asarray(grad, np.float64)
    m = beta * np.asarray(mom, np.float64) + (1.0 - beta) * grad
    return m, ((1.0 - beta) * grad + beta * m) if nesterov else m


def muon_update(w, x, lr: float, wd: float):
    """W (1 - lr wd) - lr X."""
    return np.asarray(w, np.float64) * (1.0 - lr * wd) - lr * np.asarray(x, np.float64)


def adamw(w, grad, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
          wd: float):
    """One AdamW step (step counts from 1): returns (w, m, v)."""
    g = np.asarray(grad, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    w = np.asarray(w, np.float64) * (1.0 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return w, m, v
