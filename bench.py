"""Benchmark of the GPT training step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d12]
    python bench.py --workload decode [--config d12gqa] [--decode-batch 64]
    python bench.py --workload fp8 [--config d24]
    python bench.py --workload muon [--config d12]
    python bench.py --workload optim [--config d12]
    python bench.py --workload extras [--config d12]

Times K forward+backward steps of the d12 model (12 layers, width 768, 6
heads of 128, vocab 32768, 16 rows of 2048 tokens, 'SSSL' windows 1024/2048,
value embeddings on odd layers) on synthetic seeded inputs already resident
in HBM, then prints one JSON line.  After the timed steps it runs a few more
steps with the library's launch recording on (two HIP events per kernel
launch, on the stream the kernel runs on) and reports, per kernel, the
average launch duration and the algorithmic work the library attributes to
it; the kernel with the largest share of the step is set against its
roofline.  HBM traffic of that kernel comes from the rocprofv3 counter
summary in profiles/ when the kernel's sources still hash to the value
recorded there (else null).  The CPU oracle is timed on a bounded sample of
the same workload as a reported baseline.

With --workload decode it instead times the attention of one generation
step: one new token for each of --decode-batch sequences whose caches hold
seq_len positions, every layer over its own cache with that layer's window;
the line reports new tokens/s and the KV-cache bytes read per second.
With --workload fp8 it times the step's linear layers (forward and both
backward products) as FP8 linear layers with tensor-wise scales, casts
included, beside the same products in bf16.  With --workload muon it times
Muon's Newton-Schulz orthogonalization of an update for every block matrix.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12         # bytes/s
METRIC = "train tokens/s (fwd+bwd) d12 T=2048 on 1 GPU; % bf16 MFMA peak; eval tok/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(T: int, W: int) -> int:
    """Number of (query, key) pairs with 0 <= i - j <= W in one row."""
    W = min(W, T - 1)
    # query i sees min(i, W) + 1 keys
    return sum(min(i, W) + 1 for i in range(T))


def window_of(cfg, l):
    pat = cfg["window_pattern"]
    if not pat:
        return cfg["seq_len"]
    return cfg["window_short"] if pat[l % len(pat)] == "S" else cfg["window_long"]


def model_flops(cfg):
    """Algorithmic FLOPs per token: 6 x matmul parameters + 3 x attention
    forward FLOPs over visible pairs; eval: 2 x matmul params + attention fwd."""
    D, H, Hkv, hd, V, F = (cfg["d_model"], cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"],
                           cfg["vocab"], cfg["mlp_mult"] * cfg["d_model"])
    T, L = cfg["seq_len"], cfg["n_layer"]
    mm = L * ((H + 2 * Hkv) * hd * D + D * H * hd + 2 * F * D) + V * D
    pairs = sum(visible_pairs(T, window_of(cfg, l)) for l in range(L))
    attn_fwd_per_tok = 4 * hd * H * pairs / T
    return 6 * mm + 3 * attn_fwd_per_tok, 2 * mm + attn_fwd_per_tok, mm


def time_events(fn, iters, torch):
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    st.record()
    for _ in range(iters):
        fn()
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) / iters / 1e3


def kernel_table(cfg, torch, G, iters=10):
    """Average duration of every kernel shape the step launches, timed one
    shape at a time through the kernel entry points."""
    B, T, D, H, Hkv, hd, V = (cfg["batch"], cfg["seq_len"], cfg["d_model"], cfg["n_head"],
                              cfg["n_kv_head"], cfg["head_dim"], cfg["vocab"])
    F, N, L = cfg["mlp_mult"] * D, B * T, cfg["n_layer"]
    QKV, HD = (H + 2 * Hkv) * hd, H * hd
    dev = "cuda"
    bf = torch.bfloat16
    chunk = min(N, (512 << 20) // (V * 4) // 256 * 256)
    # operand buffers sized for the largest use (checked before each launch)
    act = (torch.randn(N * max(F, QKV), device=dev) * 0.1).to(bf)        # [N, <=F] activations
    wts = (torch.randn(V * D, device=dev) * 0.02).to(bf)                 # any weight matrix
    dz = (torch.randn(N * V, device=dev, dtype=torch.float32) * 1e-5).to(bf)  # [N, V]
    out32 = torch.empty(max(chunk * V, V * D, F * D), device=dev, dtype=torch.float32)
    out16 = torch.empty(N * max(F, QKV), device=dev, dtype=bf)
    aux = torch.empty(N * F, device=dev, dtype=bf)
    rows = []
    nS = sum(1 for l in range(L) if window_of(cfg, l) < T - 1)
    gemms = [
        # name, op, M, N, K, epi, launches per step, A, B
        ("qkv_fwd NT", G.GEMM_NT, N, QKV, D, G.EPI_STORE, L, act, wts),
        ("o_fwd NT+res", G.GEMM_NT, N, D, HD, G.EPI_RESADD, L, act, wts),
        ("fc_fwd NT+relu2", G.GEMM_NT, N, F, D, G.EPI_RELU2, L, act, wts),
        ("proj_fwd NT+res", G.GEMM_NT, N, D, F, G.EPI_RESADD, L, act, wts),
        ("lm_fwd NT f32", G.GEMM_NT, chunk, V, D, G.EPI_F32, N // chunk, act, wts),
        ("lm_dx NN", G.GEMM_NN, N, D, V, G.EPI_STORE, 1, dz, wts),
        ("lm_dw TN", G.GEMM_TN, V, D, N, G.EPI_F32, 1, dz, act),
        ("proj_dw TN", G.GEMM_TN, D, F, N, G.EPI_F32, L, act, act),
        ("proj_dx NN+drelu2", G.GEMM_NN, N, F, D, G.EPI_DRELU2, L, act, wts),
        ("fc_dw TN", G.GEMM_TN, F, D, N, G.EPI_F32, L, act, act),
        ("fc_dx NN", G.GEMM_NN, N, D, F, G.EPI_STORE, L, act, wts),
        ("o_dw TN", G.GEMM_TN, D, HD, N, G.EPI_F32, L, act, act),
        ("o_dx NN", G.GEMM_NN, N, HD, D, G.EPI_STORE, L, act, wts),
        ("qkv_dw TN", G.GEMM_TN, QKV, D, N, G.EPI_F32, L, act, act),
        ("qkv_dx NN", G.GEMM_NN, N, D, QKV, G.EPI_STORE, L, act, wts),
    ]
    for name, op, M, Nn, K, epi, count, A, Bm in gemms:
        lda = K if op != G.GEMM_TN else M
        ldb = K if op == G.GEMM_NT else Nn
        f32 = epi in (G.EPI_F32, G.EPI_F32_ACC)
        Cb = out32 if f32 else out16
        need_a = (K if op == G.GEMM_TN else M) * lda
        need_b = (Nn if op == G.GEMM_NT else K) * ldb
        if A.numel() < need_a or Bm.numel() < need_b or Cb.numel() < M * Nn or \
                (epi in (G.EPI_RELU2, G.EPI_DRELU2) and aux.numel() < M * Nn):
            raise RuntimeError(f"bench buffer too small for {name}")
        sb = G.k_gemm_scratch_bytes(M, Nn, K) if f32 else 0
        scr = torch.empty(max(sb, 16), device=dev, dtype=torch.uint8) if sb else None
        fn = lambda: G.k_gemm(op, M, Nn, K, A, lda, Bm, ldb, Cb, Nn, epi,
                              aux if epi == G.EPI_DRELU2 else None, G.BF16,
                              scratch=scr)
        t = time_events(fn, iters, torch)
        rows.append(dict(kernel="gemm " + name, avg_s=t, count=count, flops=2.0 * M * Nn * K,
                         bound="mfma"))
    del act, wts, dz, out32, out16, aux
    torch.cuda.empty_cache()
    # attention (one short-window and one long-window layer shape)
    qkv = (torch.randn(N, QKV, device=dev) * 0.3).to(bf)
    o = torch.empty(N, HD, device=dev, dtype=bf)
    lse = torch.empty(B * H * T, device=dev, dtype=torch.float32)
    do = (torch.randn(N, HD, device=dev) * 0.3).to(bf)
    dqkv = torch.empty_like(qkv)
    scr = torch.empty(G.k_attn_bwd_scratch_bytes(B, T, H, hd), device=dev, dtype=torch.uint8)
    for W, count in ((cfg["window_short"], nS), (cfg["window_long"], L - nS)):
        if count == 0:
            continue
        fl = 4.0 * hd * H * B * visible_pairs(T, W)
        t = time_events(lambda: G.k_attn_fwd(qkv, o, lse, B, T, H, Hkv, hd, W, G.BF16), iters, torch)
        rows.append(dict(kernel=f"attn_fwd W={W}", avg_s=t, count=count, flops=fl, bound="mfma"))
        t = time_events(lambda: G.k_attn_bwd(qkv, o, lse, do, dqkv, scr, B, T, H, Hkv, hd, W,
                                             G.BF16), max(2, iters // 2), torch)
        rows.append(dict(kernel=f"attn_bwd W={W}", avg_s=t, count=count, flops=2 * fl,
                         bound="mfma"))
    del qkv, o, do, dqkv, scr
    torch.cuda.empty_cache()
    return rows


def kernel_profile(step, n_steps, torch, G):
    """Per-kernel time and work over n_steps steps run with the library's
    launch recording on: {name: dict(...)} per step."""
    from rocprof_summary import short_name
    torch.cuda.synchronize()
    G.prof_start(65536)
    for _ in range(n_steps):
        step()
    overflow = G.prof_stop()
    torch.cuda.synchronize()
    recs = G.prof_records()
    G.prof_clear()
    if overflow:
        raise RuntimeError("launch recording overflowed")
    agg = {}
    for name, ms, fl, by in recs:
        k = short_name(name)
        a = agg.setdefault(k, dict(kernel=k, launches=0, ms=0.0, flops=0.0, bytes=0.0))
        a["launches"] += 1
        a["ms"] += ms
        a["flops"] += fl
        a["bytes"] += by
    rows = []
    for a in agg.values():
        n = a["launches"]
        sec = a["ms"] / 1e3
        rows.append(dict(kernel=a["kernel"], launches_per_step=n / n_steps,
                         ms_per_step=a["ms"] / n_steps, avg_launch_ms=a["ms"] / n,
                         flops_per_launch=a["flops"] / n, bytes_per_launch=a["bytes"] / n,
                         tflops=a["flops"] / sec / 1e12 if a["flops"] else None,
                         gbps=a["bytes"] / sec / 1e9 if a["bytes"] else None))
    rows.sort(key=lambda r: -r["ms_per_step"])
    return rows


def roofline_of(row, step_ms, peak_flops=PEAK_BF16):
    """Roofline object of one kernel row of kernel_profile (its measured
    HBM traffic is attached by emit(), which knows the workload)."""
    sec = row["avg_launch_ms"] / 1e3
    if row["flops_per_launch"] > 0:
        ach, peak, unit, bound = row["flops_per_launch"] / sec / 1e12, peak_flops / 1e12, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = row["bytes_per_launch"] / sec / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
    return {"bound": bound, "kernel": row["kernel"], "achieved": round(ach, 2), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4),
            "traffic": None, "traffic_source": None,
            "algorithmic_flops_per_launch": row["flops_per_launch"],
            "algorithmic_bytes_per_launch": row["bytes_per_launch"],
            "avg_launch_ms": round(row["avg_launch_ms"], 4),
            "launches_per_step": row["launches_per_step"],
            "share_of_step": round(row["ms_per_step"] / step_ms, 3)}


def emit(out):
    """Print the JSON line, with the roofline kernel's HBM traffic per
    launch from the committed rocprofv3 summary of the same kernel sources
    and the same workload (null when there is none)."""
    from rocprof_summary import load_traffic
    rf = out.get("roofline")
    if rf:
        tr = load_traffic(rf["kernel"], out.get("config", {}).get("workload"))
        rf["traffic"] = tr["traffic_bytes"] if tr else None
        rf["traffic_source"] = tr["summary"] if tr else None
    print(json.dumps(out), flush=True)


def copy_calibration(torch):
    """A device copy of exactly 1 GiB (1 GiB read, 1 GiB written), three
    times, for calibrating the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copied 1 GiB x3")


def cpu_baseline(cfg, seconds_hint=10.0, max_rows=8):
    """The oracle (fp32 mode) on successive one-row batches of the workload
    until about `seconds_hint` seconds of CPU work: tokens/s."""
    import numpy as np
    import gptinputs as gi
    import oracle as O
    c1 = dict(cfg, batch=1)
    n = O.param_count(c1)
    w, _ = gi.make_params(c1, n)
    tok = gi.make_tokens(cfg, max_rows)
    rows, dt = 0, 0.0
    while rows < max_rows and (rows == 0 or dt < seconds_hint):
        t0 = time.perf_counter()
        O.step(c1, w, tok[rows:rows + 1], "fp32")
        dt += time.perf_counter() - t0
        rows += 1
    host = host_cpu_info()
    return {"value": round(rows * cfg["seq_len"] / dt, 2), "unit": "tokens/s",
            "cores": host["blas_threads"] or host["cores"], "kind": "oracle",
            "cpu_model": host["cpu_model"], "host_cores": host["cores"],
            "blas": host["blas"], "blas_threads": host["blas_threads"],
            "sample": f"{rows} one-row batches of {cfg['seq_len']} tokens from the "
                      f"{cfg['name']} workload (fwd+bwd, numpy fp32, {dt:.1f} s; the "
                      f"oracle's elementwise work is single-threaded, its products use "
                      f"the BLAS threads)"}


def host_cpu_info():
    """CPU model, usable cores and numpy's BLAS library / thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        import numpy as np
        import threadpoolctl
        np.ones(4) @ np.ones(4)
        for info in threadpoolctl.threadpool_info():
            if info.get("user_api") == "blas":
                blas = f"{info.get('internal_api')} {info.get('version')}"
                threads = int(info.get("num_threads"))
                break
    except Exception:
        pass
    return {"cpu_model": model, "cores": len(os.sched_getaffinity(0)), "blas": blas,
            "blas_threads": threads}


def gpu_clock_mhz():
    """Current shader clock (MHz) of the first AMD GPU, read from sysfs (the
    files rocm-smi reads; no child process is started), or None."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "freq1_input"))):
            try:
                with open(hw) as f:
                    return int(f.read().strip()) // 1000000
            except (OSError, ValueError):
                pass
        try:
            with open(os.path.join(dev, "pp_dpm_sclk")) as f:
                c = parse_sclk(f.read())
            if c:
                return c
        except OSError:
            pass
    return None


def parse_sclk(text):
    """The active level (marked '*') of a pp_dpm_sclk listing, in MHz, or
    None."""
    import re
    for line in text.splitlines():
        if "*" in line:
            m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
            if m:
                return int(m.group(1))
    return None


class ClockSampler:
    """Samples the shader clock every `period` seconds in a thread while
    the timed steps run; reports the median of the samples."""

    def __init__(self, period=0.5):
        import threading
        self.period, self.samples = period, []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            c = gpu_clock_mhz()
            if c:
                self.samples.append(c)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=30)

    def median(self):
        import statistics
        return statistics.median(self.samples) if self.samples else None


DECODE_METRIC = "decode attention: new tokens/s over KV caches (all layers), HBM GB/s"


def decode_inputs_gpu(torch, B, T, H, Hkv, n_layer, seed):
    """Per layer: q [B, 1, H, 128] and cached k [B, T, Hkv, 128] with unit-RMS
    rows (as after QK-norm), v N(0, 1), bf16, drawn on the device from a
    seeded generator; every cache full (length T)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)

    def unit_rms(shape):
        x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        return (x * torch.rsqrt(x.square().mean(-1, keepdim=True) + 1e-5)).bfloat16()

    layers = []
    for _ in range(n_layer):
        q = unit_rms((B, 1, H, 128))
        k = unit_rms((B, T, Hkv, 128))
        v = torch.randn((B, T, Hkv, 128), generator=g, device="cuda").bfloat16()
        layers.append((q, k, v))
    return layers


def cpu_decode_baseline(cfg, T, n_seq=32):
    """The oracle's decode attention over every layer's window for n_seq
    sequences of the workload (numpy fp32): new tokens/s."""
    import numpy as np
    import oracle as O
    from oracle.gpt import _Num
    rng = np.random.default_rng(7)
    H, Hkv = cfg["n_head"], cfg["n_kv_head"]
    dt = 0.0
    for l in range(cfg["n_layer"]):
        q = rng.standard_normal((n_seq, 1, H, 128), dtype=np.float32)
        k = rng.standard_normal((n_seq, T, Hkv, 128), dtype=np.float32)
        v = rng.standard_normal((n_seq, T, Hkv, 128), dtype=np.float32)
        t0 = time.perf_counter()
        O.decode_attention(q, k, v, np.full(n_seq, T), window_of(cfg, l), _Num("fp32"))
        dt += time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else len(os.sched_getaffinity(0))
    return {"value": round(n_seq / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_seq} sequences x {T} cached positions, all {cfg['n_layer']} layers "
                      f"(numpy fp32, {dt:.1f} s)"}


def bench_decode(a, torch, G):
    """One decode step's attention (one new token per sequence, every layer
    over its own full cache with the layer's window) timed over a.steps
    steps; roofline of the dominant launch in HBM bytes."""
    import gptinputs as gi
    cfg = gi.preset(a.config)
    T, H, Hkv, n_layer = cfg["seq_len"], cfg["n_head"], cfg["n_kv_head"], cfg["n_layer"]
    B = a.decode_batch
    log(f"decode inputs: {n_layer} layers x {B} seq x {T} positions")
    layers = decode_inputs_gpu(torch, B, T, H, Hkv, n_layer, seed=cfg["seed"])
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    outs = [(torch.empty(B, 1, H, 128, dtype=torch.bfloat16, device="cuda"),
             torch.empty(B, H, 1, dtype=torch.float32, device="cuda")) for _ in range(n_layer)]
    nbs = [G.k_attn_decode_scratch_bytes(B, 1, H, Hkv, T, window_of(cfg, l))
           for l in range(n_layer)]
    scr = torch.zeros(max(16, max(nbs)), dtype=torch.uint8, device="cuda")
    bound = 1.01 * math.sqrt(128)

    def step():
        for l, (q, k, v) in enumerate(layers):
            o, lse = outs[l]
            G.k_attn_decode(q, k, v, lens, o, lse, B, 1, T, H, Hkv, 128, window_of(cfg, l),
                            bound, scr, G.BF16)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    for o, _ in outs:
        assert torch.isfinite(o.float()).all()
    ms = time_events(step, a.steps, torch) * 1e3
    tok_s = B / (ms / 1e3)
    kv_bytes = sum(2.0 * B * min(T, window_of(cfg, l) + 1) * Hkv * 128 * 2
                   for l in range(n_layer))
    log(f"decode step {ms * 1e3:.1f} us  {tok_s:,.0f} tok/s  {kv_bytes / ms / 1e6:,.0f} GB/s")
    prof = kernel_profile(step, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    for r in prof:
        log(f"  {r['ms_per_step'] * 1e3:8.1f} us/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {r['gbps'] or 0:7.0f} GB/s  {r['kernel']}")
    roof = roofline_of(prof[0], ms) if prof else None
    cpu = None if a.no_cpu else cpu_decode_baseline(cfg, T)
    out = {
        "metric": DECODE_METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded unit-RMS q, k and N(0,1) v, full caches)",
        "config": {"workload": f"{a.config} decode attention: {B} sequences x {T} cached "
                               f"positions, 1 new token each, {n_layer} layers "
                               f"'{cfg['window_pattern']}' {cfg['window_short']}/"
                               f"{cfg['window_long']}, {H} heads on {Hkv} KV heads x 128",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU",
                   "streams": "one" if a.one_stream else
                              "two (weight-gradient work of the backward on a second stream)"},
        "kv_bytes_per_step": kv_bytes, "kv_gbps": round(kv_bytes / ms / 1e6, 1),
        "roofline": roof, "cpu_baseline": cpu,
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
    }
    emit(out)


FP8_METRIC = "FP8 (tensor-wise) linear layers fwd+bwd of a training step: tokens/s; % fp8 MFMA peak"
PEAK_FP8 = 5.0e15         # MI355X dense fp8 MFMA, FLOP/s


def linear_shapes(cfg):
    """(in, out) of the four linear layers of one block."""
    D, H, Hkv, hd = cfg["d_model"], cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    F = cfg["mlp_mult"] * D
    return [(D, (H + 2 * Hkv) * hd), (H * hd, D), (D, F), (F, D)]


def bench_fp8(a, torch, G):
    """The linear layers of one d12 step as FP8 linear layers with tensor-wise
    scales, forward and backward: per layer and linear, cast x (e4m3, with
    its transpose), cast W (e4m3, with its transpose), y = x W^T; cast dY
    (e5m2, with its transpose), dX = dY W, dW = dY^T X (fp32).  The same
    products in bf16 are timed beside it."""
    import gptinputs as gi
    cfg = gi.preset(a.config)
    N = cfg["batch"] * cfg["seq_len"]
    shapes = linear_shapes(cfg)
    L = cfg["n_layer"]
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg["seed"])
    dev = "cuda"

    def rnd(shape, scale):
        return (torch.randn(shape, generator=g, device=dev) * scale).bfloat16()

    log(f"fp8 inputs: {L} layers x {len(shapes)} linears, {N} tokens")
    lay = []
    for _ in range(L):
        for (fi, fo) in shapes:
            lay.append(dict(fi=fi, fo=fo, x=rnd((N, fi), 1.0), w=rnd((fo, fi), 0.02),
                            dy=rnd((N, fo), 1e-3)))
    u8 = torch.uint8
    mx_in = max(fi for fi, _ in shapes)
    mx_out = max(fo for _, fo in shapes)
    qx, qxt = torch.empty(N * mx_in, dtype=u8, device=dev), torch.empty(N * mx_in, dtype=u8,
                                                                          device=dev)
    qw, qwt = (torch.empty(mx_in * mx_out, dtype=u8, device=dev) for _ in range(2))
    qd, qdt = torch.empty(N * mx_out, dtype=u8, device=dev), torch.empty(N * mx_out, dtype=u8,
                                                                           device=dev)
    sc = torch.empty(12, dtype=torch.float32, device=dev)
    cscr = torch.empty(G.k_fp8_cast_scratch_bytes(), dtype=u8, device=dev)
    y = torch.empty(N * mx_out, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(N * mx_in, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(mx_in * mx_out, dtype=torch.float32, device=dev)
    gs = max(max(G.k_gemm_fp8_scratch_bytes(fo, fi, N), G.k_gemm_scratch_bytes(fo, fi, N))
             for fi, fo in shapes)
    gscr = torch.empty(max(16, gs), dtype=u8, device=dev)
    E4, E5 = G.FP8_E4M3, G.FP8_E5M2

    def step_fp8():
        for d in lay:
            fi, fo = d["fi"], d["fo"]
            G.k_fp8_cast(d["x"], N, fi, G.BF16, E4, qx, qxt, sc[0:2], cscr)
            G.k_fp8_cast(d["w"], fo, fi, G.BF16, E4, qw, qwt, sc[4:6], cscr)
            G.k_gemm_fp8(N, fo, fi, qx, fi, E4, qw, fi, E4, sc[1:2], sc[5:6], y, fo, G.EPI_STORE)
            G.k_fp8_cast(d["dy"], N, fo, G.BF16, E5, qd, qdt, sc[8:10], cscr)
            G.k_gemm_fp8(N, fi, fo, qd, fo, E5, qwt, fo, E4, sc[9:10], sc[5:6], dx, fi,
                         G.EPI_STORE)
            G.k_gemm_fp8(fo, fi, N, qdt, N, E5, qxt, N, E4, sc[9:10], sc[1:2], dw, fi, G.EPI_F32,
                         gscr)

    def step_bf16():
        for d in lay:
            fi, fo = d["fi"], d["fo"]
            G.k_gemm(G.GEMM_NT, N, fo, fi, d["x"], fi, d["w"], fi, y, fo, G.EPI_STORE, None, G.BF16)
            G.k_gemm(G.GEMM_NN, N, fi, fo, d["dy"], fo, d["w"], fi, dx, fi, G.EPI_STORE, None,
                     G.BF16)
            G.k_gemm(G.GEMM_TN, fo, fi, N, d["dy"], fo, d["x"], fi, dw, fi, G.EPI_F32, None,
                     G.BF16, scratch=gscr)

    for _ in range(a.warmup):
        step_fp8()
        step_bf16()
    torch.cuda.synchronize()
    assert torch.isfinite(y[:N * shapes[-1][1]].float()).all()
    ms8 = time_events(step_fp8, a.steps, torch) * 1e3
    ms16 = time_events(step_bf16, a.steps, torch) * 1e3
    flops = 6.0 * N * sum(fi * fo for fi, fo in shapes) * L
    log(f"fp8 linears {ms8:.3f} ms ({flops / ms8 / 1e9:,.0f} TFLOP/s incl. casts)  "
        f"bf16 {ms16:.3f} ms ({flops / ms16 / 1e9:,.0f} TFLOP/s)")
    prof = kernel_profile(step_fp8, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    for r in prof:
        rate = (f"{r['tflops']:7.1f} TFLOP/s" if r["tflops"] else
                f"{r['gbps']:7.0f} GB/s" if r["gbps"] else "")
        log(f"  {r['ms_per_step']:7.3f} ms/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {rate:>16}  {r['kernel']}")
    roof = roofline_of(prof[0], ms8, peak_flops=PEAK_FP8) if prof else None
    out = {
        "metric": FP8_METRIC, "value": round(N / (ms8 / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms8, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, N(0,1e-3) "
                "output gradients)",
        "config": {"workload": f"{a.config} linear layers fwd+bwd in FP8: {L} layers x "
                               f"{len(shapes)} linears {shapes} (in, out), {N} tokens; "
                               "e4m3 x and W, e5m2 dY, tensor-wise scales, casts included",
                   "global_batch": cfg["batch"], "seq_len": cfg["seq_len"],
                   "parallelism": "single GPU"},
        "bf16_ms_per_step": round(ms16, 4), "speedup_vs_bf16": round(ms16 / ms8, 3),
        "linear_flops_per_step": flops,
        "roofline": roof, "cpu_baseline": None if a.no_cpu else cpu_fp8_baseline(cfg),
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
    }
    emit(out)


def cpu_fp8_baseline(cfg, rows=256):
    """The oracle's FP8 linear (cast both operands, fp64 product) over every
    linear of one block for `rows` tokens, forward only: tokens/s."""
    import numpy as np
    from oracle import fp8
    rng = np.random.default_rng(1)
    dt = 0.0
    for fi, fo in linear_shapes(cfg):
        x = rng.standard_normal((rows, fi), dtype=np.float32)
        w = rng.standard_normal((fo, fi), dtype=np.float32) * 0.02
        t0 = time.perf_counter()
        fp8.fp8_linear(x, w)
        dt += time.perf_counter() - t0
    scale = cfg["n_layer"] * 3        # all layers, and the two backward products
    threads = os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else len(os.sched_getaffinity(0))
    return {"value": round(rows / (dt * scale), 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} tokens through the 4 linears of one block (forward: casts and "
                      f"fp64 product, numpy, {dt:.2f} s measured), time scaled x{scale} for "
                      f"{cfg['n_layer']} layers x 3 products of equal size"}


MUON_METRIC = "Muon orthogonalization of every matrix update of a step: ms/step; TFLOP/s"
NS_TUPLE = (3.4445, -4.7750, 2.0315)   # the classic quintic tuple, five steps


def matrix_shapes(cfg):
    """[out, in] of the matrices Muon updates: the four linears of every block."""
    return [(fo, fi) for fi, fo in linear_shapes(cfg)] * cfg["n_layer"]


def cpu_muon_baseline(shapes, coeffs):
    """The oracle's Newton-Schulz iteration (numpy fp64) on one block's
    matrices, scaled to all of them: ms per optimizer step."""
    import numpy as np
    from oracle import muon
    rng = np.random.default_rng(2)
    t0 = time.perf_counter()
    for m, n in shapes[:4]:
        muon.polar_express(rng.standard_normal((m, n)), coeffs)
    t = time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else len(os.sched_getaffinity(0))
    return {"value": round(t * len(shapes) / 4 * 1e3, 1), "unit": "ms/step", "cores": cores,
            "kind": "oracle",
            "sample": f"one block's 4 matrices (numpy fp64, {t:.2f} s measured), time scaled "
                      f"x{len(shapes) // 4}"}


def cpu_optim_baseline(muon_shapes, adam_sizes, coeffs):
    """The oracle's optimizer step (Muon momentum, Newton-Schulz and update
    for one block's matrices; AdamW for 2^20 parameters), scaled to the
    whole model: ms per step."""
    import numpy as np
    from oracle import muon
    rng = np.random.default_rng(3)
    t0 = time.perf_counter()
    for m, n in muon_shapes[:4]:
        g = rng.standard_normal((m, n))
        _, u = muon.muon_momentum(g, np.zeros_like(g), 0.95)
        muon.muon_update(np.zeros_like(g), muon.polar_express(u, coeffs), 0.02, 0.0)
    t_muon = time.perf_counter() - t0
    k = 1 << 20
    g = rng.standard_normal(k)
    t0 = time.perf_counter()
    muon.adamw(np.zeros(k), g, np.zeros(k), np.zeros(k), 1, 3e-3, 0.8, 0.95, 1e-10, 0.0)
    t_adam = time.perf_counter() - t0
    total = t_muon * len(muon_shapes) / 4 + t_adam * sum(adam_sizes) / k
    threads = os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else len(os.sched_getaffinity(0))
    return {"value": round(total * 1e3, 1), "unit": "ms/step", "cores": cores, "kind": "oracle",
            "sample": f"one block's 4 matrices through Muon ({t_muon:.2f} s) and 2^20 AdamW "
                      f"parameters ({t_adam:.3f} s), times scaled to the model"}


def bench_muon(a, torch, G):
    """Newton-Schulz orthogonalization (5 quintic steps) of a random fp32
    update for every block matrix of the model: one batched call per
    parameter shape (that parameter of every layer)."""
    import gptinputs as gi
    cfg = gi.preset(a.config)
    shapes = matrix_shapes(cfg)
    groups = sorted(set(shapes))
    L = cfg["n_layer"]
    steps = 5
    coeffs = [NS_TUPLE] * steps
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg["seed"])
    grads = [torch.randn(L, m, n, generator=g, device="cuda") for m, n in groups]
    outs = [torch.empty(L, m, n, dtype=torch.bfloat16, device="cuda") for m, n in groups]
    ws = torch.empty(max(G.k_polar_express_ws_bytes(m, n, L) for m, n in groups),
                     dtype=torch.uint8, device="cuda")

    def step():
        for (m, n), gr, o in zip(groups, grads, outs):
            G.k_polar_express(gr, m, n, G.F32, coeffs, 1e-7, o, ws, batch=L)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    assert all(torch.isfinite(o.float()).all() for o in outs)
    ms = time_events(step, a.steps, torch) * 1e3
    # per step: X^T X and X B' (2 m n^2 each) and A A (2 n^3), n the smaller side
    flops = sum(steps * (4.0 * max(m, n) * min(m, n) ** 2 + 2.0 * min(m, n) ** 3)
                for m, n in shapes)
    log(f"muon: {len(shapes)} matrices, {ms:.3f} ms per step, {flops / ms / 1e9:,.0f} TFLOP/s")
    prof = kernel_profile(step, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    for r in prof[:10]:
        rate = (f"{r['tflops']:7.1f} TFLOP/s" if r["tflops"] else
                f"{r['gbps']:7.0f} GB/s" if r["gbps"] else "")
        log(f"  {r['ms_per_step']:7.3f} ms/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {rate:>16}  {r['kernel']}")
    roof = roofline_of(prof[0], ms) if prof else None
    cpu = None if a.no_cpu else cpu_muon_baseline(shapes, coeffs)
    out = {
        "metric": MUON_METRIC, "value": round(ms, 4), "unit": "ms/step", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 updates)",
        "config": {"workload": f"{a.config} Muon orthogonalization: {len(shapes)} matrices, "
                               f"{L} of each of {groups} batched per call, {steps} quintic "
                               f"Newton-Schulz steps {NS_TUPLE}", "parallelism": "single GPU"},
        "tflops": round(flops / ms / 1e9, 1), "ns_flops_per_step": flops,
        "roofline": roof, "cpu_baseline": cpu,
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
    }
    emit(out)


OPTIM_METRIC = "optimizer step (Muon for block matrices, AdamW for the rest): ms/step"


def bench_optim(a, torch, G):
    """One optimizer step over every parameter of the model (gpt_optim_step):
    Muon (momentum, batched Newton-Schulz per parameter shape, update with a
    bf16 copy) for the block matrices, AdamW for the embeddings, lm_head,
    value embeddings and gates; fp32 masters, gradients and states resident
    in HBM."""
    import gptinputs as gi
    cfg = gi.preset(a.config)
    if a.one_stream:
        cfg["one_stream"] = 1
    gc = G.make_config(cfg)
    L = cfg["n_layer"]
    n_total = G.param_count(gc)
    D, F, V = cfg["d_model"], cfg["mlp_mult"] * cfg["d_model"], cfg["vocab"]
    H, Hkv, hd, C = cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"], cfg["ve_gate_channels"]
    shape_of = {G.P_WQKV: ((H + 2 * Hkv) * hd, D), G.P_WO: (D, H * hd), G.P_WFC: (F, D),
                G.P_WPROJ: (D, F), G.P_VE: (V, Hkv * hd), G.P_WG: (Hkv, C)}
    groups = {}
    adam = [(G.param_offset(gc, G.P_WTE), (V, D)), (G.param_offset(gc, G.P_WLM), (V, D))]
    for l in range(L):
        for p in (G.P_WQKV, G.P_WO, G.P_WFC, G.P_WPROJ):
            groups.setdefault(p, []).append((G.param_offset(gc, p, l), shape_of[p]))
        for p in (G.P_VE, G.P_WG):
            off = G.param_offset(gc, p, l)
            if off >= 0:
                adam.append((off, shape_of[p]))
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(cfg["seed"])
    w = torch.randn(n_total, generator=g, device=dev) * 0.02
    w16 = w.bfloat16()
    grad = torch.randn(n_total, generator=g, device=dev) * 1e-3
    mom, m2 = torch.zeros(n_total, device=dev), torch.zeros(n_total, device=dev)
    hp = G.make_optim_hparams([NS_TUPLE] * 5)
    ows = torch.empty(G.optim_ws_bytes(gc), dtype=torch.uint8, device=dev)
    coeffs = [NS_TUPLE] * 5

    def numel(shape):
        return int(math.prod(shape))

    def step():
        G.optim_step(gc, hp, 1, w, w16, grad, mom, m2, ows)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    assert torch.isfinite(w).all()
    ms = time_events(step, a.steps, torch) * 1e3
    n_muon = sum(numel(s) for v in groups.values() for _, s in v)
    log(f"optimizer step {ms:.3f} ms: {n_muon:,} Muon + {n_total - n_muon:,} AdamW parameters")
    # per-kernel split with every group on one stream (a kernel's time then
    # carries no overlap with the groups on the library's side streams)
    gc_one = G.make_config(dict(cfg, one_stream=1))

    def step_one():
        G.optim_step(gc_one, hp, 1, w, w16, grad, mom, m2, ows)

    prof = kernel_profile(step_one, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    for r in prof[:10]:
        rate = (f"{r['tflops']:7.1f} TFLOP/s" if r["tflops"] else
                f"{r['gbps']:7.0f} GB/s" if r["gbps"] else "")
        log(f"  {r['ms_per_step']:7.3f} ms/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {rate:>16}  {r['kernel']}")
    roof = roofline_of(prof[0], ms) if prof else None
    out = {
        "metric": OPTIM_METRIC, "value": round(ms, 4), "unit": "ms/step", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "fp32+bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1e-3) gradients)",
        "config": {"workload": f"{a.config} optimizer step: {n_muon} Muon parameters in "
                               f"{len(groups)} shape groups of {L} (momentum 0.95 Nesterov, 5 "
                               f"quintic Newton-Schulz steps), {n_total - n_muon} AdamW "
                               "parameters", "parallelism": "single GPU",
                   "streams": "one" if a.one_stream else
                              "four (Muon groups beside each other and AdamW)"},
        "roofline": roof,
        "cpu_baseline": None if a.no_cpu else cpu_optim_baseline(
            [s for v in groups.values() for _, s in v[:1]] * L,
            [numel(s) for _, s in adam], coeffs),
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
    }
    emit(out)


EXTRAS_METRIC = "model extras (smear, residual lambdas, backout) fwd+bwd of a step: GB/s"


def bench_extras(a, torch, G):
    """The model extras of one training step at the workload's token count:
    smear once after the embedding, residual mixing before every block,
    backout once after the last; forward and backward of each."""
    import gptinputs as gi
    cfg = gi.preset(a.config)
    B, T, D, L = cfg["batch"], cfg["seq_len"], cfg["d_model"], cfg["n_layer"]
    N = B * T
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(cfg["seed"])

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device=dev).bfloat16()

    x0, xs, dy = rnd(N, D), [rnd(N, D) for _ in range(L)], rnd(N, D)
    xm = rnd(N, D)
    y, dx, dx0 = (torch.empty(N, D, dtype=torch.bfloat16, device=dev) for _ in range(3))
    lam = torch.tensor([0.9, 0.1], device=dev).bfloat16()
    bo = torch.tensor([1.0, -0.3], device=dev).bfloat16()
    w = rnd(24)
    sl = torch.tensor([0.5], device=dev).bfloat16()
    gate = torch.empty(N, device=dev)
    dl = torch.empty(32, device=dev)
    mscr = torch.empty(G.lib().gpt_k_resid_mix_bwd_scratch_bytes(), dtype=torch.uint8, device=dev)
    sscr = torch.empty(G.lib().gpt_k_smear_bwd_scratch_bytes(), dtype=torch.uint8, device=dev)
    n = N * D

    def step():
        G.k_smear_fwd(x0, B, T, D, w, sl, y, gate, G.BF16)
        for x in xs:
            G.k_resid_mix_fwd(x, x0, y, n, lam, G.BF16)
        G.k_resid_mix_fwd(y, xm, dx, n, bo, G.BF16)
        G.k_resid_mix_bwd(dy, y, xm, None, dx0, False, n, bo, dl[0:], mscr, G.BF16)
        for x in xs:
            G.k_resid_mix_bwd(dy, x, x0, dx, dx0, True, n, lam, dl[2:], mscr, G.BF16)
        G.k_smear_bwd(dy, x0, B, T, D, w, sl, gate, dx, dl[4:], sscr, G.BF16)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, a.steps, torch) * 1e3
    # bytes: smear fwd 3 nD (x, x_prev, y) + bwd 4 nD; mix fwd 3 nD, bwd 5 nD (dy, x, x0, dx,
    # dx0 read and written: 6); backout fwd 3, bwd 4 -- bf16, 2 bytes each
    per = 2.0 * n
    nbytes = per * (3 + 4 + L * (3 + 6) + 3 + 4)
    gbs = nbytes / ms / 1e6
    log(f"extras {ms:.3f} ms per step, {gbs:,.0f} GB/s")
    prof = kernel_profile(step, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    for r in prof[:8]:
        log(f"  {r['ms_per_step']:7.3f} ms/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {r['gbps'] or 0:7.0f} GB/s  {r['kernel']}")
    roof = roofline_of(prof[0], ms) if prof else None
    out = {
        "metric": EXTRAS_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and gradients)",
        "config": {"workload": f"{a.config} model extras: smear + backout once, residual "
                               f"mixing x {L}, forward and backward, {N} tokens x {D}",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU",
                   "streams": "one" if a.one_stream else
                              "two (weight-gradient work of the backward on a second stream)"},
        "roofline": roof, "cpu_baseline": None,
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
    }
    emit(out)


EVAL_BATCH_TOKENS = 131072


def eval_batch_rows(cfg, n_rows):
    """Rows per gpt_eval_bpb batch: up to 131,072 tokens (64 d12 rows, 32
    d12-GQA rows), at least the training batch.  Larger batches fill the
    GEMMs' rounds of 256 tiles better (d12, 64 rows: 3.41M tokens/s against
    3.25M in batches of 16); the result does not depend on the batching."""
    return max(cfg["batch"], min(n_rows, EVAL_BATCH_TOKENS // cfg["seq_len"]))


def eval_set_line(name, torch, G, gi, Session, iters=2):
    """Evaluation tokens/s and bpb of a preset over its whole evaluation set
    (gpt_eval_bpb calls over the set, `iters` of them timed with events
    after one warm-up call)."""
    cfg = gi.preset(name)
    _, eval_fpt, _ = model_flops(cfg)
    n_rows = cfg["eval_rows"]
    cfg["batch"] = eval_batch_rows(cfg, n_rows)
    s = Session(cfg, eval_ws=True, train_ws=False)
    w, bits = gi.make_params(cfg, s.n_params)
    s.set_params(w, bits)
    del w, bits
    tok = s.upload(gi.make_eval_tokens(cfg, n_rows))
    tb = s.upload(gi.make_token_bytes(cfg))
    s.evaluate(tok, tb)
    torch.cuda.synchronize()
    t = time_events(lambda: s.evaluate(tok, tb), iters, torch)
    targets = n_rows * cfg["seq_len"]
    bpb = s.bpb.cpu().numpy().tolist()
    log(f"{name} eval over {targets} targets: {targets / t:,.0f} tok/s, bpb {bpb[2]:.4f}")
    out = {"workload": f"{name} evaluation set: {n_rows} rows x {cfg['seq_len']} "
                       f"({targets} targets), batches of {cfg['batch']}",
           "tokens_per_s": round(targets / t, 1), "seconds": round(t, 4), "bpb": bpb[2],
           "mfu_bf16": round(targets / t * eval_fpt / PEAK_BF16, 4)}
    del s, tok, tb
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None,
                    help="preset (train: d12, decode: d12gqa, fp8: d24)")
    ap.add_argument("--eval-rows", type=int, default=64)
    ap.add_argument("--prof-steps", type=int, default=2,
                    help="steps run with launch recording for the per-kernel split (0: none)")
    ap.add_argument("--shapes", action="store_true",
                    help="also time every product / attention shape alone")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gqa-eval", action="store_true",
                    help="train: skip the evaluation-set lines (d12-GQA over 2^21 targets, "
                         "d24 over 2^22)")
    ap.add_argument("--one-stream", action="store_true",
                    help="train: the whole step on one stream (no second stream for the "
                         "weight-gradient work); optim: every Muon group on one stream")
    ap.add_argument("--workload", choices=("train", "decode", "fp8", "muon", "optim", "extras"),
                    default="train",
                    help="train: the fwd+bwd step; decode: KV-cache decode attention; fp8: the "
                         "step's linear layers as FP8 linear layers; muon: Muon's "
                         "orthogonalization of every matrix update; optim: the whole optimizer "
                         "step; extras: smear, residual lambdas and backout")
    ap.add_argument("--model-extras", action="store_true",
                    help="train: turn on residual mixing, smear and backout (after the middle "
                         "block) inside the step")
    ap.add_argument("--decode-batch", type=int, default=64,
                    help="sequences sampled in parallel (decode workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB device copy used to calibrate HBM counters")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the step is built and "
              "measured on one GPU's share, see the design notes for how it would shard",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import gptinputs as gi
    import gpt_pretraining_step_amd as G
    from gpt_pretraining_step_amd.session import Session

    torch.cuda.set_device(0)
    if a.copy_calibration:
        copy_calibration(torch)
        return
    if a.workload == "decode":
        a.config = a.config or "d12gqa"
        bench_decode(a, torch, G)
        return
    if a.workload == "extras":
        a.config = a.config or "d12"
        bench_extras(a, torch, G)
        return
    if a.workload == "optim":
        a.config = a.config or "d12"
        bench_optim(a, torch, G)
        return
    if a.workload == "muon":
        a.config = a.config or "d12"
        bench_muon(a, torch, G)
        return
    if a.workload == "fp8":
        a.config = a.config or "d24"
        bench_fp8(a, torch, G)
        return
    a.config = a.config or "d12"
    cfg = gi.preset(a.config)
    if a.model_extras:
        cfg.update(resid_lambdas=1, smear=1, backout_layer=cfg["n_layer"] // 2)
    if a.one_stream:
        cfg.update(one_stream=1)
    train_fpt, eval_fpt, mm = model_flops(cfg)
    B, T = cfg["batch"], cfg["seq_len"]
    tokens_per_step = B * T

    log("building inputs", a.config)
    s = Session(cfg)
    w, bits = gi.make_params(cfg, s.n_params)
    if a.model_extras:
        # the extras vector's slots (C ABI layout): mixing weights (1, 0.1)
        # per block, smear lambda 0.5, backout lambda 0.2
        L, off = cfg["n_layer"], G.param_offset(s.cfg, G.P_EXTRAS)
        w[off:off + 2 * L:2], w[off + 1:off + 2 * L:2] = 1.0, 0.1
        w[off + 2 * L + 24], w[off + 2 * L + 25] = 0.5, 0.2
        bits = gi.bf16_bits_from_f32(w)
        w = gi.f32_from_bf16_bits(bits)
    s.set_params(w, bits)
    s.set_tokens(gi.make_tokens(cfg))
    del w, bits

    def step():
        s.fwd()
        s.bwd()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    loss0 = s.loss.item()
    assert math.isfinite(loss0), loss0
    log(f"warmup done, loss {loss0:.4f}")
    # one event before each step and one after the last, on the stream the
    # library's kernels run on: K per-step times, and the whole span
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        evs[0].record()
        for k in range(a.steps):
            step()
            evs[k + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per_step = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(a.steps)])
    ms_mean = evs[0].elapsed_time(evs[-1]) / a.steps
    ms = float(np.median(per_step))
    p10, p90 = (float(np.percentile(per_step, q)) for q in (10, 90))
    tok_s = tokens_per_step / (ms / 1e3)
    mfu = tok_s * train_fpt / PEAK_BF16
    clock = clk.median()
    max_clock = 2400
    mfu_clk = mfu * max_clock / clock if clock else None
    log(f"step median {ms:.2f} ms (p10 {p10:.2f}, p90 {p90:.2f}, mean {ms_mean:.2f})  "
        f"{tok_s:,.0f} tok/s  mfu {mfu:.3f}  clock {clock} MHz  (wall {wall:.2f} s)")

    # the optimizer step on the same model (fp32 masters and states), timed
    # on its own: reported beside the fwd+bwd rate, not folded into it
    opt = {}
    for normuon in (False, True):
        hp = G.make_optim_hparams([NS_TUPLE] * 5, normuon=normuon)
        master = s.params.float()
        st1, st2 = torch.zeros_like(master), torch.zeros_like(master)
        ows = torch.empty(G.optim_ws_bytes(s.cfg), dtype=torch.uint8, device="cuda")
        opt_params = s.params.clone()
        G.optim_step(s.cfg, hp, 1, master, opt_params, s.grads, st1, st2, ows)
        torch.cuda.synchronize()
        opt[normuon] = time_events(lambda: G.optim_step(s.cfg, hp, 2, master, opt_params,
                                                        s.grads, st1, st2, ows), 5, torch) * 1e3
        del master, st1, st2, ows, opt_params
        torch.cuda.empty_cache()
    opt_ms = opt[False]
    log(f"optimizer step {opt_ms:.2f} ms (NorMuon {opt[True]:.2f} ms); fwd+bwd+optimizer "
        f"{tokens_per_step / ((ms + opt_ms) / 1e3):,.0f} tok/s")

    # evaluation throughput (forward + CE + bytes reduction), in batches of
    # eval_batch_rows rows (a session of that batch sharing the parameters)
    ev_rows = a.eval_rows
    ev_batch = eval_batch_rows(cfg, ev_rows)
    se = Session(dict(cfg, batch=ev_batch), eval_ws=True, train_ws=False)
    se.params = s.params
    ev_tok = se.upload(gi.make_eval_tokens(cfg, ev_rows))
    tb = se.upload(gi.make_token_bytes(cfg))
    se.evaluate(ev_tok, tb)
    torch.cuda.synchronize()
    t_ev = time_events(lambda: se.evaluate(ev_tok, tb), 2, torch)
    eval_tok_s = ev_rows * T / t_ev
    bpb = se.bpb.cpu().numpy().tolist()
    log(f"eval {eval_tok_s:,.0f} tok/s (batches of {ev_batch} rows), bpb {bpb[2]:.4f}")
    del ev_tok, se
    torch.cuda.empty_cache()
    # the long-context workload's evaluation: d12-GQA over its whole 2^21-
    # target set (512 rows x 4096), a separate model of that shape
    gqa = d24 = None
    if not a.model_extras and a.config == "d12" and not a.no_gqa_eval:
        gqa = eval_set_line("d12gqa", torch, G, gi, Session)
        # and d24's 2^22-target set (about 7 s a pass: one timed pass)
        d24 = eval_set_line("d24", torch, G, gi, Session, iters=1)

    # per-kernel split of the step with the library's launch recording, the
    # step on one stream (a kernel's time then carries no overlap with the
    # backward's second stream)
    step_cfg = s.cfg
    s.cfg = G.make_config(dict(cfg, one_stream=1))
    prof = kernel_profile(step, a.prof_steps, torch, G) if a.prof_steps > 0 else []
    s.cfg = step_cfg
    roof = roofline_of(prof[0], ms) if prof else None
    for r in prof[:14]:
        rate = (f"{r['tflops']:7.1f} TFLOP/s" if r["tflops"] else
                f"{r['gbps']:7.0f} GB/s" if r["gbps"] else "")
        log(f"  {r['ms_per_step']:7.3f} ms/step {r['launches_per_step']:5.0f} x "
            f"{r['avg_launch_ms'] * 1e3:8.1f} us  {rate:>16}  {r['kernel']}")
    if roof:
        log(f"roofline: {roof['kernel']} {roof['achieved']} {roof['unit']} "
            f"frac {roof['frac']} traffic {roof['traffic']}")

    table = []
    if a.shapes:
        del s
        torch.cuda.empty_cache()
        table = kernel_table(cfg, torch, G)
        for r in table:
            r["tflops"] = r["flops"] / r["avg_s"] / 1e12
            log(f"  {r['kernel']:<24} {r['avg_s'] * 1e3:8.3f} ms x{r['count']:<3} "
                f"{r['tflops']:7.1f} TFLOP/s")

    cpu = None if a.no_cpu else cpu_baseline(cfg)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 3),
        "ms_per_step_stats": {"median": round(ms, 3), "p10": round(p10, 3),
                              "p90": round(p90, 3), "mean": round(ms_mean, 3),
                              "value_from": "median"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) random-init weights)",
        "config": {"workload": f"{a.config} fwd+bwd step: {cfg['n_layer']} layers, "
                               f"d_model {cfg['d_model']}, {cfg['n_head']}x{cfg['head_dim']} "
                               f"heads ({cfg['n_kv_head']} KV), vocab {cfg['vocab']}, "
                               f"{B} rows x T={T} ({tokens_per_step} tokens), windows "
                               f"'{cfg['window_pattern']}' {cfg['window_short']}/"
                               f"{cfg['window_long']}, value embeddings on odd layers"
                               + (f", model extras (residual mixing, smear, backout after "
                                  f"block {cfg['backout_layer']})" if a.model_extras else ""),
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU",
                   "streams": "one" if a.one_stream else
                              "two (weight-gradient work of the backward on a second stream)"},
        "mfu_bf16": round(mfu, 4), "train_flop_per_token": train_fpt,
        "gpu_clock_mhz": clock, "mfu_bf16_clock_adjusted": round(mfu_clk, 4) if mfu_clk else None,
        "clock_note": f"median shader clock read from sysfs during the timed steps; "
                      f"the adjusted MFU prices the peak at that clock instead of "
                      f"{max_clock} MHz",
        "optimizer_ms_per_step": round(opt_ms, 3),
        "optimizer_ms_per_step_normuon": round(opt[True], 3),
        "optimizer_ns": f"Muon Newton-Schulz: {NS_TUPLE} x 5 (the classic quintic tuple; the "
                        f"page prints two of its five tuples)",
        "tokens_per_s_with_optimizer": round(tokens_per_step / ((ms + opt_ms) / 1e3), 1),
        "eval_tokens_per_s": round(eval_tok_s, 1), "eval_rows": ev_rows,
        "eval_batch_rows": ev_batch, "eval_bpb": bpb[2],
        "eval_mfu_bf16": round(eval_tok_s * eval_fpt / PEAK_BF16, 4),
        "eval_d12gqa_2m": gqa, "eval_d24_4m": d24,
        "context": {
            "autoresearch_5min_budget": {
                "d12_steps_in_300s": int(300.0 / (ms / 1e3)),
                "d12_tokens_in_300s": int(300.0 / (ms / 1e3)) * tokens_per_step,
                "d12_steps_in_300s_with_optimizer": int(300.0 / ((ms + opt_ms) / 1e3)),
                "note": "the autoresearch pages give each experiment 5 minutes of training "
                        "on one GPU"},
            "microgpt_cpu": "the microgpt page's pure-Python run: 1,000 steps of a "
                            "4,192-parameter model in about a minute on a CPU"},
        "roofline": roof, "cpu_baseline": cpu,
        "kernels": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                    for r in prof],
        "shapes": [{k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()}
                   for r in table],
    }
    emit(out)


if __name__ == "__main__":
    main()
