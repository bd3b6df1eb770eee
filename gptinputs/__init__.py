"""Seeded synthetic inputs for the compact GPT training step.

This module is shared by the CPU oracle tests and the GPU path's tests and
benchmark.  It holds configuration presets (shapes only) and seeded random
generators for weights, token rows and per-vocabulary byte lengths.  It holds
none of the model's arithmetic: nothing here normalises, rotates, attends,
projects or reduces.

Workload recipe (one seed root per preset, numpy SeedSequence):
    root.spawn(4) -> [params, train tokens, eval tokens, byte table]

* weights: every weight entry is sigma * N(0, 1), drawn as float32 standard
  normals from numpy's PCG64 Generator; bf16 presets then round each value to
  the nearest bf16 (ties to even).  sigma = 0.08 for the tiny character model,
  0.02 otherwise.  Whole flat parameter buffer, one draw.
* tiny tokens: column 0 is BOS (id 0), the other columns uniform in 1..26
  (a 27-symbol character vocabulary, microgpt's letters + BOS).
* other presets: every position i.i.d. from a Zipf(s=1.1) law truncated to the
  vocabulary, P(id = r-1) proportional to r^-1.1, by inverse CDF.  This stands
  in for BPE-tokenised web text, whose unigram law is Zipf-like.
* byte table: tiny -> all ones; others -> uniform in 1..8 per vocabulary id.
  This stands in for the bytes-per-token of a real BPE vocabulary, which the
  bits-per-byte metric divides by.

Each token row holds T+1 ids: inputs are the first T, targets the last T.
"""
from __future__ import annotations

import copy
import numpy as np

__all__ = [
    "PRESETS", "preset", "make_params", "make_tokens", "make_eval_tokens",
    "make_token_bytes", "bf16_bits_from_f32", "f32_from_bf16_bits",
]

DTYPE_F32 = 0
DTYPE_BF16 = 1

_BASE = dict(mlp_mult=4, ve_gate_channels=32, rope_base=10000.0,
             norm_eps=1e-5, ve_every_odd=1)

# Shapes and distributions of the five workloads.  The d<depth> presets follow
# the depth dial: width = 64 * depth, heads = width / 128.
PRESETS = {
    "tiny": dict(_BASE, n_layer=1, d_model=16, n_head=4, n_kv_head=2,
                 head_dim=4, vocab=27, seq_len=16, batch=8,
                 window_pattern="", window_short=0, window_long=0,
                 ve_every_odd=0, dtype=DTYPE_F32, sigma=0.08, seed=0,
                 tokens="chars", eval_rows=8),
    "d4": dict(_BASE, n_layer=4, d_model=256, n_head=2, n_kv_head=2,
               head_dim=128, vocab=8192, seq_len=512, batch=16,
               window_pattern="SL", window_short=256, window_long=512,
               dtype=DTYPE_BF16, sigma=0.02, seed=4, tokens="zipf",
               eval_rows=16),
    "d12": dict(_BASE, n_layer=12, d_model=768, n_head=6, n_kv_head=6,
                head_dim=128, vocab=32768, seq_len=2048, batch=16,
                window_pattern="SSSL", window_short=1024, window_long=2048,
                dtype=DTYPE_BF16, sigma=0.02, seed=12, tokens="zipf",
                eval_rows=16),
    "d12gqa": dict(_BASE, n_layer=12, d_model=768, n_head=6, n_kv_head=2,
                   head_dim=128, vocab=32768, seq_len=4096, batch=8,
                   window_pattern="SSSL", window_short=1024, window_long=4096,
                   dtype=DTYPE_BF16, sigma=0.02, seed=1204, tokens="zipf",
                   eval_rows=512),      # 512 x 4096 = 2^21 eval targets
    "d24": dict(_BASE, n_layer=24, d_model=1536, n_head=12, n_kv_head=12,
                head_dim=128, vocab=32768, seq_len=2048, batch=16,
                window_pattern="SSSL", window_short=1024, window_long=2048,
                dtype=DTYPE_BF16, sigma=0.02, seed=24, tokens="zipf",
                eval_rows=2048),     # 2048 x 2048 = 2^22 eval targets
}


def preset(name: str, **overrides) -> dict:
    """A copy of a preset with fields overridden (e.g. batch=2)."""
    cfg = copy.deepcopy(PRESETS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def _streams(cfg: dict):
    return np.random.SeedSequence(int(cfg["seed"])).spawn(4)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def make_params(cfg: dict, n_params: int):
    """Flat weights for a preset.

    Returns (values_f32, bf16_bits_or_None).  For bf16 presets values_f32
    holds exactly the bf16 values (so both sides of a comparison see the same
    numbers); for fp32 presets the bits entry is None.
    """
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[0]))
    w = rng.standard_normal(n_params, dtype=np.float32)
    w *= np.float32(cfg["sigma"])
    if cfg["dtype"] == DTYPE_BF16:
        bits = bf16_bits_from_f32(w)
        return f32_from_bf16_bits(bits), bits
    return w, None


def _zipf_cdf(vocab: int, s: float = 1.1) -> np.ndarray:
    r = np.arange(1, vocab + 1, dtype=np.float64)
    p = r ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def _draw_rows(cfg: dict, rng: np.random.Generator, n_rows: int) -> np.ndarray:
    T1 = cfg["seq_len"] + 1
    if cfg["tokens"] == "chars":
        t = rng.integers(1, 27, size=(n_rows, T1), dtype=np.int64)
        t[:, 0] = 0
        return t.astype(np.int32)
    cdf = _zipf_cdf(cfg["vocab"])
    u = rng.random(size=(n_rows, T1))
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, cfg["vocab"] - 1).astype(np.int32)


def make_tokens(cfg: dict, n_rows: int | None = None) -> np.ndarray:
    """Training rows [n_rows, T+1] int32 (default: the preset's batch)."""
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[1]))
    return _draw_rows(cfg, rng, cfg["batch"] if n_rows is None else n_rows)


def make_eval_tokens(cfg: dict, n_rows: int | None = None) -> np.ndarray:
    """Evaluation rows [n_rows, T+1] from a stream separate from training.

    Rows are drawn in order, so the first k rows of a larger draw equal a
    draw of k rows.
    """
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[2]))
    return _draw_rows(cfg, rng, cfg["eval_rows"] if n_rows is None else n_rows)


def make_token_bytes(cfg: dict) -> np.ndarray:
    """Per-vocabulary byte lengths int32 [V]."""
    if cfg["tokens"] == "chars":
        return np.ones(cfg["vocab"], dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[3]))
    return rng.integers(1, 9, size=cfg["vocab"], dtype=np.int64).astype(np.int32)
