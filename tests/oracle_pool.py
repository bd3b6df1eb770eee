"""The oracle over many rows at once, in worker processes (test infrastructure).

Rows are independent in the model (attention never crosses rows, everything
else is per token), so the gradient of a batch's mean loss is the mean of
the rows' own gradients, and a batch's evaluation sums are the sums of its
rows'.  The oracle is single-threaded for most of its work, so the rows run
in parallel processes: each worker maps the weights from one file, runs
`oracle.step` (or `oracle.eval_bpb`) on its rows and writes its partial sum.
Workers start by spawning (they never inherit a GPU context) and import
only numpy, the oracle and the input generators.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np


def cpu_share(limit: int = 16) -> int:
    """Cores this process may use, at most `limit` (a GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _grad_worker(args):
    cfg, wpath, tok, prec, outpath = args
    import oracle as O
    w = np.load(wpath, mmap_mode="r")
    gsum, losses = None, []
    for row in tok:
        loss, g, _ = O.step(dict(cfg, batch=1), w, row[None], prec)
        g = np.asarray(g, np.float32)
        if gsum is None:
            gsum = g.copy()
        else:
            gsum += g
        losses.append(float(loss))
    np.save(outpath, gsum)
    return losses


def _eval_worker(args):
    cfg, wpath, tok, tb, prec = args
    import oracle as O
    w = np.load(wpath, mmap_mode="r")
    out = []
    for row in tok:
        r = O.eval_bpb(dict(cfg, batch=1), w, row[None], tb, prec)
        out.append((float(r[0]), float(r[1])))
    return out


def _pool_run(fn, jobs, workers, threads):
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                         "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = str(threads)
    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            return pool.map(fn, jobs)
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _split(rows, workers):
    workers = max(1, min(workers, len(rows)))
    return [rows[i::workers] for i in range(workers)]


def mean_row_gradients(cfg, w, tokens, prec="bf16emu", workers=None, cores=None):
    """(mean over rows of the rows' gradients (fp32), per-row losses), the
    oracle run on every row of tokens [B, T+1] as a one-row batch."""
    cores = cores or cpu_share()
    rows = list(range(tokens.shape[0]))
    parts = _split(rows, workers or cores)
    threads = max(1, cores // len(parts))
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        wpath = os.path.join(tmp, "w.npy")
        np.save(wpath, np.asarray(w, np.float32))
        jobs = [(dict(cfg), wpath, np.ascontiguousarray(tokens[p]), prec,
                 os.path.join(tmp, f"g{i}.npy")) for i, p in enumerate(parts)]
        losses_by_part = _pool_run(_grad_worker, jobs, len(parts), threads)
        total = None
        for i in range(len(parts)):
            g = np.load(os.path.join(tmp, f"g{i}.npy"))
            total = g.astype(np.float64) if total is None else total + g
        losses = np.empty(len(rows))
        for p, ls in zip(parts, losses_by_part):
            losses[p] = ls
        return total / len(rows), losses
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def row_eval_sums(cfg, w, tokens, token_bytes, prec="bf16emu", workers=None, cores=None):
    """Per row of tokens [R, T+1]: (sum of nats, sum of bytes), float64 [R, 2]."""
    cores = cores or cpu_share()
    rows = list(range(tokens.shape[0]))
    parts = _split(rows, workers or cores)
    threads = max(1, cores // len(parts))
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        wpath = os.path.join(tmp, "w.npy")
        np.save(wpath, np.asarray(w, np.float32))
        jobs = [(dict(cfg), wpath, np.ascontiguousarray(tokens[p]), token_bytes, prec)
                for p in parts]
        res = _pool_run(_eval_worker, jobs, len(parts), threads)
        out = np.empty((len(rows), 2))
        for p, r in zip(parts, res):
            out[p] = r
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
