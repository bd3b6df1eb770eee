"""Launch recording (gpt_prof_*): every launch of a step is recorded with
its kernel name, a positive duration and the work the library attributes to
it."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gptinputs as gi  # noqa: E402
import gpt_pretraining_step_amd as G  # noqa: E402
from gpt_pretraining_step_amd.session import Session  # noqa: E402
from rocprof_summary import short_name  # noqa: E402
from tests.gpu_util import small_bf16  # noqa: E402


def test_gemm_launch_is_recorded_with_its_flops():
    M, N, K = 512, 384, 256
    a = (torch.randn(M, K, device="cuda") * 0.1).to(torch.bfloat16)
    b = (torch.randn(N, K, device="cuda") * 0.1).to(torch.bfloat16)
    c = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    G.prof_start(16)
    G.k_gemm(G.GEMM_NT, M, N, K, a, K, b, K, c, N, G.EPI_STORE, None, G.BF16)
    assert G.prof_stop() is False
    recs = G.prof_records()
    G.prof_clear()
    assert len(recs) == 1
    name, ms, fl, by = recs[0]
    assert short_name(name).startswith("k_gemm_mfma")
    assert ms > 0
    assert fl == 2.0 * M * N * K
    assert by == 2.0 * (M * K + N * K) + 2.0 * M * N
    torch.testing.assert_close(c.float(), (a.float() @ b.float().T), atol=2e-2, rtol=2e-2)


def test_step_launches_recorded_and_overflow_flagged():
    cfg = small_bf16()
    s = Session(cfg)
    w, bits = gi.make_params(cfg, s.n_params)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    G.prof_start(4096)
    s.fwd()
    s.bwd()
    assert G.prof_stop() is False
    recs = G.prof_records()
    names = {short_name(r[0]) for r in recs}
    assert len(recs) > 5 * cfg["n_layer"]
    assert all(r[1] >= 0 for r in recs)
    assert any(n.startswith("k_attn") for n in names)
    assert any(n.startswith("k_gemm") for n in names)
    # a capacity below the launch count is reported, never overrun
    G.prof_start(3)
    s.fwd()
    assert G.prof_stop() is True
    assert len(G.prof_records()) == 3
    G.prof_clear()
    assert G.lib().gpt_prof_count() == 0
