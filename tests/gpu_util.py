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


def grads_by_tensor(cfg, flat):
    out, off = {}, 0
    for name, shape in O.param_layout(cfg):
        n = int(np.prod(shape))
        out[name] = np.asarray(flat[off:off + n]).reshape(shape)
        off += n
    return out
