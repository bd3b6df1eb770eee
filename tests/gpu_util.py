"""Helpers shared by the GPU parity tests (no model arithmetic here)."""
import numpy as np

import gptinputs as gi
import oracle as O


def rel_err(got, ref) -> float:
    """Normwise max relative error: max|got - ref| / max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy() if t.dtype != torch.float64 \
        else t.detach().cpu().numpy()


def small_bf16(**kw):
    """A small bf16 model with every feature on (windows, GQA, value
    embeddings), sized so the oracle takes a second or two."""
    d = gi.preset("d4", n_layer=2, d_model=128, n_head=2, n_kv_head=1, head_dim=64,
                  vocab=500, seq_len=96, batch=3, window_pattern="SL", window_short=16,
                  window_long=96, ve_gate_channels=32, seed=77)
    d.update(kw)
    return d


def tiny_plus():
    return gi.preset("tiny", n_layer=2, window_pattern="SL", window_short=4,
                     window_long=16, ve_every_odd=1, ve_gate_channels=8)


def set_extras(cfg, w, seed=5):
    """Put plausible values in the extras slots of a flat vector (in place):
    resid lambdas near 1, x0 lambdas near 0.3, small smear weights, smear
    lambda 0.6, backout lambda 0.35; padding zero."""
    if not O.extras_on(cfg):
        return w
    sl = O.extras_slots(cfg)
    off = O.param_count(cfg) - sl["size"]
    rng = np.random.default_rng(seed)
    ex = np.zeros(sl["size"])
    L = cfg["n_layer"]
    ex[0:2 * L:2] = 1.0 + 0.2 * rng.standard_normal(L)
    ex[1:2 * L:2] = 0.3 + 0.1 * rng.standard_normal(L)
    ex[sl["smear_w"]:sl["smear_w"] + 24] = 0.5 * rng.standard_normal(24)
    ex[sl["smear_lambda"]] = 0.6
    ex[sl["backout"]] = 0.35
    w[off:off + sl["size"]] = ex
    return w


def with_extras(cfg, w, bits):
    """(values, bf16 bits or None) of a flat vector whose extras slots hold
    set_extras' values, rounded to bf16 for bf16 configs so both sides see
    the same numbers."""
    w = set_extras(cfg, np.asarray(w, np.float32).copy())
    if bits is None:
        return w, None
    b = gi.bf16_bits_from_f32(w)
    return gi.f32_from_bf16_bits(b), b


def grads_by_tensor(cfg, flat):
    out, off = {}, 0
    for name, shape in O.param_layout(cfg):
        n = int(np.prod(shape))
        out[name] = np.asarray(flat[off:off + n]).reshape(shape)
        off += n
    return out
