"""Writes tests/golden/eval_sums.json: the oracle's evaluation sums on
sampled full-size batches of the evaluation sets (test infrastructure).

    python tests/golden/make_eval_golden.py [--workers N] [--only d12,d24]

For each workload: the preset (shapes, seed), which batches were taken
(rows [b B, (b + 1) B) of the seeded evaluation set), and per batch the
oracle's (sum of nats, sum of bytes) in its bf16-emulation mode (float64
sums), the rounding points of the bf16 GPU path.  Only the oracle and the
seeded input generators run here; the GPU path never writes these values.

Batches:
  d12     the 64 rows the benchmark's evaluation line runs (4 batches of 16)
  d12gqa  batches 0, 21, 42, 63 of the 2^21-target set (64 batches of 8 x 4096)
  d24     batches 0, 42, 85, 127 of the 2^22-target set (128 batches of 16 x 2048)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gptinputs as gi  # noqa: E402
import oracle as O  # noqa: E402
from tests import oracle_pool  # noqa: E402

OUT = os.path.join(HERE, "eval_sums.json")
SAMPLES = {"d12": (64, [0, 1, 2, 3]), "d12gqa": (None, [0, 21, 42, 63]),
           "d24": (None, [0, 42, 85, 127])}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=None)
    ap.add_argument("--only", default="")
    a = ap.parse_args(argv)
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    names = [n for n in SAMPLES if not a.only or n in a.only.split(",")]
    for name in names:
        t0 = time.time()
        cfg = gi.preset(name)
        n_rows, batches = SAMPLES[name]
        n_rows = n_rows or cfg["eval_rows"]
        B = cfg["batch"]
        w, _ = gi.make_params(cfg, O.param_count(cfg))
        tok = gi.make_eval_tokens(cfg, n_rows)
        tb = gi.make_token_bytes(cfg)
        rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in batches])
        sums = oracle_pool.row_eval_sums(cfg, w, tok[rows], tb, "bf16emu", workers=a.workers)
        per = sums.reshape(len(batches), B, 2).sum(axis=1)
        data[name] = {
            "preset": {k: v for k, v in cfg.items()},
            "eval_rows": n_rows, "rows_per_batch": B, "precision": "bf16emu",
            "batches": {str(b): [float(per[i, 0]), float(per[i, 1])]
                        for i, b in enumerate(batches)},
        }
        json.dump(data, open(OUT, "w"), indent=1, sort_keys=True)
        print(f"{name}: {len(rows)} rows in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
