"""CPU oracle of the compact GPT decoder training step -- TEST INFRASTRUCTURE.

This package is a plain, slow, obviously-correct NumPy statement of what the
GPU path computes.  It exists to check the GPU path and nothing else: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import,
call or execute it.  The product path never routes through it.

It shares no code with the HIP library; the only module both sides use is the
seeded input generator (``gptinputs``), which holds no model arithmetic.

Sources (pages, cited by title and section):
  [nanochat]  "5만원으로 나만의 ChatGPT 훈련하는 방법" (apidog.com blog, nanochat
              walkthrough): "1. GPT model (nanochat/gpt.py)" architecture list
              and efficiency tricks (`oracle.extras`),
              value-embedding snippet; "2. Muon optimizer" (the Newton-
              Schulz orthogonalization, `oracle.muon`); "3. precision
              management" (also the FP8 linear layers, `oracle.fp8`); "5. flash
              attention integration" (causal + window_size call); "6.
              inference engine" (KV-cache attention of new tokens).
  [microgpt]  "microgpt" (news.hada.io): "model architecture" (RMSNorm, ReLU,
              residual, multi-head attention), "training loop" (cross-entropy
              on the next token), "parameter initialisation" (~4,192 params).
  [autoresearch] tilnote.io autoresearch summary, "core mechanism": val_bpb,
              validation bits per byte, lower is better.

Parity status: every function here is pinned by the CPU tests (finite
differences, closed forms, invariants, brute force); see the test suite.
"""
from .gpt import (  # noqa: F401
    PRECISIONS, param_layout, param_count, unpack_params, window_for_layer,
    is_ve_layer, visible_mask, rope_tables, rope, rope_bwd, rmsnorm,
    rmsnorm_bwd, attention, attention_bwd, attention_tiled, decode_attention,
    cross_entropy,
    embedding, embedding_bwd, value_embedding, value_embedding_bwd,
    forward, backward, step, eval_bpb, round_bf16, extras_on, extras_slots,
)
from . import fp8  # noqa: F401  (FP8 linear layers with tensor-wise scaling)
from . import muon  # noqa: F401  (Muon's Newton-Schulz orthogonalization)
from . import extras  # noqa: F401  (residual lambdas, smear, backout)
