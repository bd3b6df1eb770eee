"""Device buffers for one model configuration (torch tensors as plain memory).

A Session owns the workspace, parameter, gradient, token and result buffers
of one configuration and calls the library's entry points on them.  It holds
no arithmetic of the model.
"""
from __future__ import annotations

import numpy as np

from . import (BF16, MODE_EVAL, MODE_TRAIN, eval_bpb, make_config, param_count,
               step_bwd, step_fwd, workspace_bytes, ws_offset)


class Session:
    def __init__(self, cfg: dict, device: str = "cuda", eval_ws: bool = False,
                 train_ws: bool = True):
        import torch
        self.torch = torch
        self.d = dict(cfg)
        self.cfg = make_config(cfg)
        self.device = device
        self.n_params = param_count(self.cfg)
        self.bf16 = cfg["dtype"] == BF16
        self.pdtype = torch.bfloat16 if self.bf16 else torch.float32
        self.ws = (torch.empty(workspace_bytes(self.cfg, MODE_TRAIN), dtype=torch.uint8,
                               device=device) if train_ws else None)
        self.ws_eval = (torch.empty(workspace_bytes(self.cfg, MODE_EVAL), dtype=torch.uint8,
                                    device=device) if eval_ws else None)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.bpb = torch.zeros(3, dtype=torch.float64, device=device)
        self.grads = (torch.zeros(self.n_params, dtype=torch.float32, device=device)
                      if train_ws else None)
        self.params = None
        self.tokens = None

    # -------------------------------------------------------------- inputs
    def set_params(self, values_f32: np.ndarray, bf16_bits: np.ndarray | None = None):
        torch = self.torch
        if self.bf16:
            if bf16_bits is None:
                raise ValueError("bf16 config needs the bf16 bits of the weights")
            t = torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16))
            self.params = t.view(torch.bfloat16).to(self.device)
        else:
            self.params = torch.from_numpy(np.ascontiguousarray(values_f32, np.float32)).to(self.device)

    def set_tokens(self, tokens: np.ndarray):
        self.tokens = self.torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).to(self.device)

    def upload(self, arr: np.ndarray, dtype=None):
        t = self.torch.from_numpy(np.ascontiguousarray(arr))
        return t.to(self.device) if dtype is None else t.to(self.device, dtype)

    # -------------------------------------------------------------- calls
    def fwd(self, stream=None):
        step_fwd(self.cfg, self.params, self.tokens, self.ws, self.loss, stream)

    def bwd(self, accumulate: bool = False, stream=None):
        step_bwd(self.cfg, self.params, self.tokens, self.ws, self.grads, accumulate, stream)

    def evaluate(self, tokens_dev, token_bytes_dev, stream=None):
        eval_bpb(self.cfg, self.params, tokens_dev, token_bytes_dev, self.ws_eval, self.bpb,
                 stream)

    # ---------------------------------------------------- workspace views
    def ws_f32(self, which: int, count: int, layer: int = 0):
        off = ws_offset(self.cfg, which, layer)
        return self.ws[off:off + 4 * count].view(self.torch.float32)

    def ws_act(self, which: int, count: int, layer: int = 0):
        es = 2 if self.bf16 else 4
        off = ws_offset(self.cfg, which, layer)
        return self.ws[off:off + es * count].view(self.pdtype)
