"""gpt_k_attn_decode_noalloc (decode attention with library-owned scratch)
against gpt_k_attn_decode with a caller buffer (GPU only): the same kernels
on the same inputs, so the outputs must agree bit for bit; two calls in a
row, the second smaller, then the first shape again."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gpt_pretraining_step_amd as G  # noqa: E402

DEV = "cuda"


def _inputs(B, Tq, Tmax, H, Hkv, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)

    def unit_rms(shape):
        x = torch.randn(shape, generator=g, device=DEV)
        return (x / x.pow(2).mean(-1, keepdim=True).add(1e-5).sqrt()).to(torch.bfloat16)

    q = unit_rms((B, Tq, H, 128))
    k = unit_rms((B, Tmax, Hkv, 128))
    v = torch.randn((B, Tmax, Hkv, 128), generator=g, device=DEV).to(torch.bfloat16)
    return q, k, v


def _run(noalloc, q, k, v, lens, B, Tq, Tmax, H, Hkv, W, bound):
    o = torch.full((B, Tq, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        G.k_attn_decode_noalloc(q, k, v, lens, o, lse, B, Tq, Tmax, H, Hkv, 128, W, bound,
                                G.BF16)
    else:
        nb = G.k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, W)
        scr = torch.zeros(max(nb, 16), dtype=torch.uint8, device=DEV)
        G.k_attn_decode(q, k, v, lens, o, lse, B, Tq, Tmax, H, Hkv, 128, W, bound, scr, G.BF16)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# B, Tq, Tmax, H, Hkv, window, lengths (ragged, one empty): several chunks
# per sequence, so the scratch is used
CASES = [
    (8, 1, 4096, 6, 2, 4096, [4096, 4000, 3333, 64, 65, 0, 4096, 1]),
    (2, 4, 1000, 8, 2, 700, [1000, 517]),
]


def test_noalloc_matches_caller_buffer():
    assert G.k_attn_decode_noalloc_max_scratch() == 8 << 20
    for i, (B, Tq, Tmax, H, Hkv, W, lens) in enumerate(CASES + CASES[:1]):
        need = G.k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, W)
        print("noalloc decode", (B, Tq, Tmax, H, Hkv, W), "scratch", need, flush=True)
        assert 0 < need <= G.k_attn_decode_noalloc_max_scratch()
        q, k, v = _inputs(B, Tq, Tmax, H, Hkv, seed=70 + i)
        tl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        for bound in (0.0, 1.01 * math.sqrt(128)):
            ref = _run(False, q, k, v, tl, B, Tq, Tmax, H, Hkv, W, bound)
            got = _run(True, q, k, v, tl, B, Tq, Tmax, H, Hkv, W, bound)
            assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
            assert np.array_equal(got[1].numpy(), ref[1].numpy(), equal_nan=True)
            assert torch.isfinite(got[0].float()).all()
