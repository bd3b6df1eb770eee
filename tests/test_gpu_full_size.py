"""Parity at the full model sizes of d12, d12-GQA and d24 (GPU only).

At the benchmark's launch configuration (d12: 16 rows x 2048, one step)
and at d12-GQA's (8 rows x 4096), every gradient tensor of the full-batch
step is compared with the oracle's: rows never interact, so the gradient of
the batch's mean loss is exactly the mean of the rows' own gradients, which
the oracle computes row by row in parallel worker processes
(tests/oracle_pool.py).  d24 is compared the same way on four spread rows
of its batch.  Evaluation: the benchmark's 64 d12 evaluation rows and
spread full-size batches of the 2M (d12-GQA) and 4M (d24) token sets
against sums the oracle wrote once (tests/golden/eval_sums.json, by
tests/golden/make_eval_golden.py); the GPU's sums over the whole 2M / 4M
sets must also be the sums of its per-batch results.
Bars: normwise max relative error 2e-2 against the oracle's bf16 emulation,
1e-3 absolute on bits per byte.
"""
import sys

import numpy as np
import pytest

import gptinputs as gi
import oracle as O
from tests.gpu_util import grads_by_tensor, rel_err, to_np, with_extras

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import gpt_pretraining_step_amd as G  # noqa: E402
from gpt_pretraining_step_amd.session import Session  # noqa: E402

TOL = 2e-2
NAMES = ["d12", "d12gqa", "d24", "d12+extras"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_cache = {}


def model(name):
    """Preset, oracle-side fp32 weights and the bf16 bits, cached per preset."""
    if name not in _cache:
        if name == "d12+extras":
            # the d12 step with residual mixing, smear and backout after
            # the middle block
            cfg = gi.preset("d12", resid_lambdas=1, smear=1, backout_layer=6)
        else:
            cfg = gi.preset(name)
        n = O.param_count(cfg)
        w, bits = with_extras(cfg, *gi.make_params(cfg, n))
        _cache.clear()
        _cache[name] = (cfg, w, bits)
    return _cache[name]


@pytest.mark.parametrize("name", ["d24", "d12+extras"])
def test_sampled_row_losses_at_bench_batch(name):
    cfg, w, bits = model(name)
    tok = gi.make_tokens(cfg)
    say(name, "full batch", tok.shape)
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    torch.cuda.synchronize()
    B, T = tok.shape[0], tok.shape[1] - 1
    ell = to_np(s.ws_f32(G.WS_ELL, B * T)).reshape(B, T)
    flag = int(s.ws[G.ws_offset(s.cfg, G.WS_NONFINITE):][:4].view(torch.int32).item())
    assert flag == 0
    assert abs(s.loss.item() - ell.astype(np.float64).mean()) < 1e-5
    for b in (0, B - 1):
        _, cache = O.forward(dict(cfg, batch=1), w, tok[b:b + 1], "bf16emu", keep=False)
        err = rel_err(ell[b], cache["ell"])
        say(name, "row", b, "loss rel err", f"{err:.2e}")
        assert err < TOL


# rows of the preset's training batch compared at full batch: all of them
# (d12 and d12-GQA, the launch configurations of the benchmark and of the
# long-context workload), or four spread rows as one batch (d24)
FULL_BATCH = {"d12": None, "d12gqa": None, "d24": [0, 5, 10, 15]}


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(FULL_BATCH))
def test_full_batch_gradients_vs_oracle(name):
    """Every gradient tensor of the full-batch step against the oracle's
    mean of the rows' one-row gradients (bf16 emulation), the mean loss and
    every row's mean loss against the oracle's."""
    from tests import oracle_pool
    cfg, w, bits = model(name)
    tok = gi.make_tokens(cfg)
    if FULL_BATCH[name] is not None:
        tok = np.ascontiguousarray(tok[FULL_BATCH[name]])
        cfg = dict(cfg, batch=tok.shape[0])
    B, T = tok.shape[0], tok.shape[1] - 1
    say(name, "GPU step at batch", B, "x", T)
    s = Session(cfg)
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    loss = s.loss.item()
    row_loss = to_np(s.ws_f32(G.WS_ELL, B * T)).reshape(B, T).mean(axis=1)
    got = s.grads.cpu().numpy()
    del s
    torch.cuda.empty_cache()
    say(name, "oracle over", B, "rows on", oracle_pool.cpu_share(), "cores")
    ref, ref_rows = oracle_pool.mean_row_gradients(cfg, w, tok, "bf16emu")
    say(name, "loss gpu", loss, "oracle", ref_rows.mean())
    assert abs(loss - ref_rows.mean()) / ref_rows.mean() < 1e-3
    assert np.abs(row_loss - ref_rows).max() / ref_rows.mean() < 1e-3
    g, r = grads_by_tensor(cfg, got), grads_by_tensor(cfg, ref)
    errs = {k: rel_err(g[k], r[k]) for k in r}
    worst = sorted(errs.items(), key=lambda kv: -kv[1])[:4]
    say(name, "worst grad errors", [(k, f"{v:.2e}") for k, v in worst])
    bad = {k: v for k, v in errs.items() if not v < TOL}
    assert not bad, bad


@pytest.mark.parametrize("name", ["d12+extras"])
def test_gradients_one_row_full_width(name):
    cfg, w, bits = model(name)
    c1 = dict(cfg, batch=1)
    tok = gi.make_tokens(cfg, 1)
    s = Session(c1)
    s.set_params(w, bits)
    s.set_tokens(tok)
    s.fwd()
    s.bwd()
    torch.cuda.synchronize()
    got = grads_by_tensor(c1, to_np(s.grads))
    loss = s.loss.item()
    del s
    torch.cuda.empty_cache()
    say(name, "oracle step (1 row)")
    ref_loss, ref_g, _ = O.step(c1, w, tok, "bf16emu")
    assert abs(loss - ref_loss) / ref_loss < 1e-3
    ref = grads_by_tensor(c1, ref_g)
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    worst = sorted(errs.items(), key=lambda kv: -kv[1])[:4]
    say(name, "worst grad errors", [(k, f"{v:.2e}") for k, v in worst])
    bad = {k: v for k, v in errs.items() if not v < TOL}
    assert not bad, bad


@pytest.mark.parametrize("name", ["d24"])
def test_batch_gradient_is_mean_of_row_gradients(name):
    """At d24's own batch of 16 (the oracle sees four of its rows above):
    the full-batch gradient equals the mean of the GPU's one-row
    gradients, a property of the mean loss at any size."""
    cfg, w, bits = model(name)
    tok = gi.make_tokens(cfg)
    B = tok.shape[0]
    full = Session(cfg)
    full.set_params(w, bits)
    full.set_tokens(tok)
    full.fwd()
    full.bwd()
    g_full = full.grads.clone()
    del full
    torch.cuda.empty_cache()
    one = Session(dict(cfg, batch=1))
    one.params = None
    one.set_params(w, bits)
    for b in range(B):
        one.set_tokens(tok[b:b + 1])
        one.fwd()
        one.bwd(accumulate=b > 0)
    torch.cuda.synchronize()
    mean_rows = one.grads / B
    err = rel_err(to_np(g_full), to_np(mean_rows))
    say(name, "batch vs mean-of-rows gradient rel err", f"{err:.2e}")
    assert err < 1e-2


def _golden(name):
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "eval_sums.json")
    d = json.load(open(path))[name]
    # the sums belong to this exact workload (shapes, seed)
    assert d["preset"] == {k: v for k, v in gi.preset(name).items()}
    return d


def _bpb(nats, nbytes):
    return nats / (np.log(2.0) * nbytes)


def test_eval_bench_rows_vs_oracle():
    """The benchmark's evaluation line: d12, 64 evaluation rows in batches
    of 16, per batch and in total against the oracle's sums."""
    gold = _golden("d12")
    cfg, w, bits = model("d12")
    n_rows, Bsz = gold["eval_rows"], gold["rows_per_batch"]
    tok = gi.make_eval_tokens(cfg, n_rows)
    tb = gi.make_token_bytes(cfg)
    s = Session(cfg, eval_ws=True, train_ws=False)
    s.set_params(w, bits)
    dtb, dtok = s.upload(tb), s.upload(tok)
    tot = np.zeros(2)
    for b, (nats, nbytes) in sorted(gold["batches"].items(), key=lambda kv: int(kv[0])):
        b = int(b)
        s.evaluate(dtok[b * Bsz:(b + 1) * Bsz], dtb)
        torch.cuda.synchronize()
        got = s.bpb.cpu().numpy()
        say("d12 eval batch", b, "bpb gpu", got[2], "oracle", _bpb(nats, nbytes))
        assert got[1] == nbytes
        assert abs(got[2] - _bpb(nats, nbytes)) < 1e-3
        tot += (nats, nbytes)
    s.evaluate(dtok, dtb)
    torch.cuda.synchronize()
    got = s.bpb.cpu().numpy()
    say("d12 eval 64 rows: bpb gpu", got[2], "oracle", _bpb(*tot))
    assert got[1] == tot[1] and abs(got[2] - _bpb(*tot)) < 1e-3


@pytest.mark.parametrize("name", ["d12gqa", "d24"])
def test_eval_bpb_full_set(name):
    """The whole 2M / 4M-token set on the GPU: its sums are the sums of its
    per-batch results, the bytes equal the table's count, and four spread
    full-size batches agree with the oracle's sums to 1e-3 in bpb."""
    gold = _golden(name)
    cfg, w, bits = model(name)
    Bsz = cfg["batch"]
    n_rows = cfg["eval_rows"]                 # 2M (d12-GQA) / 4M (d24) targets
    assert gold["eval_rows"] == n_rows and gold["rows_per_batch"] == Bsz
    tok = gi.make_eval_tokens(cfg, n_rows)
    tb = gi.make_token_bytes(cfg)
    s = Session(cfg, eval_ws=True, train_ws=False)
    s.set_params(w, bits)
    dtb = s.upload(tb)
    dtok = s.upload(tok)
    s.evaluate(dtok, dtb)
    torch.cuda.synchronize()
    full = s.bpb.cpu().numpy().copy()
    assert full[1] == tb[tok[:, 1:]].sum()
    nats, per = 0.0, {}
    for r0 in range(0, n_rows, Bsz):
        s.evaluate(dtok[r0:r0 + Bsz], dtb)
        torch.cuda.synchronize()
        b = s.bpb.cpu().numpy()
        per[r0 // Bsz] = b.copy()
        nats += float(b[0])
    assert abs(nats - full[0]) / full[0] < 1e-9
    for b, (onats, obytes) in gold["batches"].items():
        got = per[int(b)]
        say(name, "batch", b, "bpb gpu", got[2], "oracle", _bpb(onats, obytes))
        assert got[1] == obytes
        assert abs(got[2] - _bpb(onats, obytes)) < 1e-3
    say(name, "full set bpb", full[2])


def test_decode_attention_bench_workload():
    """KV-cache decode attention at the benchmark's decode workload and launch
    configuration (d12-GQA: 64 sequences x 4096 cached positions, one new
    token, 6 heads on 2 KV heads, score bound on): the first four layers'
    inputs ('SSSL': windows 1024 and 4096), every sequence and head against
    the oracle."""
    import math
    import bench
    from oracle.gpt import _Num
    cfg = gi.preset("d12gqa")
    B, T, H, Hkv = 64, cfg["seq_len"], cfg["n_head"], cfg["n_kv_head"]
    layers = bench.decode_inputs_gpu(torch, B, T, H, Hkv, 4, seed=cfg["seed"])
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    for l, (q, k, v) in enumerate(layers):
        W = bench.window_of(cfg, l)
        say("decode layer", l, "window", W)
        o = torch.empty(B, 1, H, 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, H, 1, dtype=torch.float32, device="cuda")
        nb = G.k_attn_decode_scratch_bytes(B, 1, H, Hkv, T, W)
        scr = torch.zeros(max(16, nb), dtype=torch.uint8, device="cuda")
        G.k_attn_decode(q, k, v, lens, o, lse, B, 1, T, H, Hkv, 128, W, 1.01 * math.sqrt(128),
                        scr, G.BF16)
        torch.cuda.synchronize()
        o_ref, lse_ref = O.decode_attention(to_np(q), to_np(k), to_np(v), np.full(B, T), W,
                                            _Num("bf16emu"))
        assert rel_err(to_np(o), o_ref) < TOL
        assert rel_err(to_np(lse), lse_ref) < 1e-5
