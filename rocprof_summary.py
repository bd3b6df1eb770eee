"""rocprofv3 summaries for profiles/, and the HBM traffic bench.py reports.

    python rocprof_summary.py --kernel NAME --stats DIR [--fetch DIR --write DIR
        --cal-fetch DIR --cal-write DIR] [--bench-json FILE] [--cmd TEXT ...]
        --out profiles/<file>.md

--stats is the output folder of a `rocprofv3 --kernel-trace --stats -f csv`
run; --fetch / --write are `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
runs (with --kernel-trace, -f csv) of the workload; --cal-fetch / --cal-write
the same counters over `bench.py --copy-calibration`, a device copy of
exactly 1 GiB (1 GiB read, 1 GiB written), which fixes the bytes each counter
unit stands for on this part.  The summary gives the per-kernel time table,
the kernel's counters per dispatch and, on a line starting `traffic-json:`,
its calibrated HBM bytes per launch with a hash of the kernel's sources;
bench.py reports that traffic only while the sources still hash the same.

    python rocprof_summary.py --table --bench-json FILE --fetch DIR --write DIR
        --cal-fetch DIR --cal-write DIR --mfma DIR [--mops COUNTER] [--waits DIR]
        [--marker KERNEL] [--peak TFLOPS] --out profiles/<file>.md

--table writes one row per kernel of the bench line's `kernels` list (launch
times from the library's HIP events): its measured HBM bytes per launch and
the rate they give against 8 TB/s, and from a `rocprofv3 --pmc MfmaUtil
<mops counter>` run the fraction of SIMD cycles its matrix cores were busy
and the MFMA rate the op counter gives (512 flops per unit) against the
dtype's peak; with --waits, from a run of the SQ wait counters, the share of
the waves' cycles spent waiting for data or barriers, for an issue slot and
for an LDS issue slot.  With --marker only the dispatches between the second
and the third launch of that kernel (one timed step) are counted.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gpt_pretraining_step_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30


def short_name(name: str) -> str:
    """'void gk::k_x<1, 2>(int, ...)' -> 'k_x<1, 2>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    return n.replace("gk::", "").strip()


def kernel_sources_sha256(kernel: str) -> str:
    """sha256 over the source file(s) defining the kernel and every header
    of the library's source folder."""
    base = re.sub(r"<.*", "", kernel)
    files = []
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith(".h"):
            files.append(f)
        elif f.endswith((".hip", ".cpp")):
            with open(f, encoding="utf-8") as fh:
                if re.search(r"\bvoid\s+" + re.escape(base) + r"\s*\(", fh.read()):
                    files.append(f)
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic(kernel: str, workload: str | None = None):
    """Calibrated HBM bytes per launch of `kernel` from profiles/, or None
    when no summary covers it, its sources changed since, or (with a
    workload) the summary was taken on another workload."""
    want = kernel_sources_sha256(kernel)
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("traffic-json:"):
                    d = json.loads(line[len("traffic-json:"):])
                    if d.get("kernel") == kernel and d.get("sources_sha256") == want and \
                            (workload is None or d.get("workload") == workload):
                        d["summary"] = os.path.relpath(f, ROOT)
                        return d
    return None


def _one(path: str, pattern: str) -> str:
    hits = glob.glob(os.path.join(path, "**", pattern), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one {pattern} under {path}, found {hits}")
    return hits[0]


def read_stats(d: str):
    rows = []
    with open(_one(d, "*kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append(dict(name=short_name(r["Name"]), calls=int(r["Calls"]),
                             total_ns=float(r["TotalDurationNs"]), avg_ns=float(r["AverageNs"]),
                             pct=float(r["Percentage"])))
    return rows


def read_counter(d: str, counter: str):
    """{short kernel name: [value per dispatch]} (KiB for *_SIZE counters)."""
    out = {}
    with open(_one(d, "*counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def read_dispatches(d: str, marker: str | None):
    """[(short kernel name, {counter: value})] in dispatch order; with a
    marker, only the dispatches from its second launch up to its third."""
    by_id = {}
    with open(_one(d, "*counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            e = by_id.setdefault(int(r["Dispatch_Id"]), (short_name(r["Kernel_Name"]), {}))
            e[1][r["Counter_Name"]] = float(r["Counter_Value"])
    seq = [by_id[i] for i in sorted(by_id)]
    if marker:
        at = [i for i, (n, _) in enumerate(seq) if n == marker]
        if len(at) < 3:
            raise SystemExit(f"{marker} launched {len(at)} times in {d}")
        seq = seq[at[1]:at[2]]
    return seq


def per_kernel_mean(seq, counter: str):
    acc = {}
    for n, c in seq:
        if counter in c:
            acc.setdefault(n, []).append(c[counter])
    return {n: sum(v) / len(v) for n, v in acc.items()}


def step_table(a):
    with open(a.bench_json) as fh:
        bench = json.loads([l for l in fh if l.startswith("{")][-1])
    ff = copy_factor(a.cal_fetch, "FETCH_SIZE")[0]
    wf = copy_factor(a.cal_write, "WRITE_SIZE")[0]
    fetch = per_kernel_mean(read_dispatches(a.fetch, a.marker), "FETCH_SIZE")
    write = per_kernel_mean(read_dispatches(a.write, a.marker), "WRITE_SIZE")
    mseq = read_dispatches(a.mfma, a.marker)
    util = per_kernel_mean(mseq, "MfmaUtil")
    mops = per_kernel_mean(mseq, a.mops)
    waits = None
    if a.waits:
        wseq = read_dispatches(a.waits, a.marker)
        waits = {c: per_kernel_mean(wseq, c) for c in
                 ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
                  "SQ_LDS_BANK_CONFLICT")}
    L = [f"# {a.title}", ""]
    if a.cmd:
        L += ["Commands (run from the repository root; rocprofv3 after "
              "`cd /tmp && export TMPDIR=/tmp`, paths shortened):", ""]
        L += [f"    {c}" for c in a.cmd] + [""]
    L += [f"Launch times: the library's HIP events over the bench line's profiled steps "
          f"({bench['config'].get('workload')}). HBM: calibrated FETCH_SIZE + WRITE_SIZE per "
          f"dispatch (factors {ff:.4f} and {wf:.4f} bytes per counted byte) over the launch "
          f"time, against 8 TB/s. MFMA busy: `MfmaUtil`, the matrix cores' busy cycles over "
          f"the SIMD cycles of the dispatch. MFMA rate: `{a.mops}` x 512 flops over the launch "
          f"time, against {a.peak:.0f} TFLOP/s; it counts every MFMA issued, recomputed "
          f"products included, while the algorithmic rate counts each result once.", "",
          "| kernel | launches / step | us / launch | algorithmic rate | HBM MB / launch "
          "| HBM GB/s (of 8 TB/s) | MFMA busy | MFMA TFLOP/s (of peak) |"
          + (" wait: data / issue / LDS issue | LDS bank conflicts |" if waits else ""),
          "|---|---:|---:|---:|---:|---:|---:|---:|" + ("---:|---:|" if waits else "")]
    if waits:
        L[-3:-3] = [f"Waits (a run of `rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_ANY "
                    f"SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT ...`): the "
                    f"fractions of the waves' cycles spent waiting for anything (data, "
                    f"barriers), for an instruction issue slot, and for an LDS issue slot; "
                    f"bank conflicts in cycles per dispatch.", ""]
    for k in bench["kernels"][:a.top]:
        n, t = k["kernel"], k["avg_launch_ms"] / 1e3
        alg = (f"{k['tflops']:.0f} TFLOP/s" if k.get("tflops") else
               f"{k['gbps']:.0f} GB/s" if k.get("gbps") else "")
        hbm = ((fetch[n] * ff + write[n] * wf) * 1024 if n in fetch and n in write else None)
        hb = f"{hbm / 1e6:.1f}" if hbm is not None else ""
        hr = f"{hbm / t / 1e9:.0f} ({hbm / t / 8e12:.0%})" if hbm is not None else ""
        mu = f"{util[n]:.1f}%" if n in util else ""
        mr = (f"{mops[n] * 512 / t / 1e12:.0f} ({mops[n] * 512 / t / 1e12 / a.peak:.0%})"
              if mops.get(n) else "")
        row = (f"| `{n}` | {k['launches_per_step']:.0f} | {t * 1e6:.1f} | {alg} | {hb} | {hr} "
               f"| {mu} | {mr} |")
        if waits:
            wc = waits["SQ_WAVE_CYCLES"].get(n)
            if wc:
                f = lambda c: waits[c].get(n, 0.0) / wc
                row += (f" {f('SQ_WAIT_ANY'):.0%} / {f('SQ_WAIT_INST_ANY'):.0%} / "
                        f"{f('SQ_WAIT_INST_LDS'):.1%} | {waits['SQ_LDS_BANK_CONFLICT'].get(n, 0):.0f} |")
            else:
                row += " | |"
        L.append(row)
    L.append("")
    with open(a.out, "w") as fh:
        fh.write("\n".join(L))
    print(a.out)


def copy_factor(d: str, counter: str):
    """Bytes per counter KiB unit, from the 1 GiB copy: the largest dispatch
    of the calibration run is the copy."""
    vals = read_counter(d, counter)
    name, best = max(((k, max(v)) for k, v in vals.items()), key=lambda kv: kv[1])
    return COPY_BYTES / (best * 1024.0), name, best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--table", action="store_true")
    ap.add_argument("--mfma")
    ap.add_argument("--waits")
    ap.add_argument("--mops", default="SQ_INSTS_VALU_MFMA_MOPS_BF16")
    ap.add_argument("--marker")
    ap.add_argument("--peak", type=float, default=2500.0)
    ap.add_argument("--kernel")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--cal-fetch")
    ap.add_argument("--cal-write")
    ap.add_argument("--bench-json")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--title", default="")
    ap.add_argument("--top", type=int, default=25)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.table:
        return step_table(a)
    if not (a.kernel and a.stats):
        ap.error("--kernel and --stats are required without --table")

    stats = read_stats(a.stats)
    tot = sum(r["total_ns"] for r in stats)
    L = [f"# {a.title or a.kernel}", ""]
    if a.cmd:
        L += ["Commands (run from the repository root; rocprofv3 after "
              "`cd /tmp && export TMPDIR=/tmp`, paths shortened):", ""]
        L += [f"    {c}" for c in a.cmd] + [""]
    bench = None
    if a.bench_json:
        with open(a.bench_json) as fh:
            lines = [l for l in fh if l.startswith("{")]
        bench = json.loads(lines[-1])
        rf = bench.get("roofline") or {}
        L += [f"bench.py line of the profiled run: {bench['value']:,.0f} {bench['unit']}, "
              f"{bench['ms_per_step']} ms/step; roofline kernel `{rf.get('kernel')}`, "
              f"avg launch {rf.get('avg_launch_ms')} ms (HIP events), achieved "
              f"{rf.get('achieved')} {rf.get('unit')}, frac {rf.get('frac')}", ""]
    L += [f"Kernel time over the whole run: {tot / 1e6:.2f} ms", "",
          "| share | total ms | calls | avg us | kernel |", "|---:|---:|---:|---:|---|"]
    for r in sorted(stats, key=lambda r: -r["total_ns"])[:a.top]:
        L.append(f"| {r['pct']:.2f}% | {r['total_ns'] / 1e6:.3f} | {r['calls']} | "
                 f"{r['avg_ns'] / 1e3:.1f} | `{r['name']}` |")
    L.append("")
    mine = [r for r in stats if r["name"] == a.kernel]
    if not mine:
        raise SystemExit(f"{a.kernel} not in {a.stats}")
    L += [f"`{a.kernel}`: {mine[0]['calls']} calls, average {mine[0]['avg_ns'] / 1e3:.1f} us "
          "(rocprofv3 kernel trace).", ""]
    if a.fetch and a.write and a.cal_fetch and a.cal_write:
        ff, fname, fval = copy_factor(a.cal_fetch, "FETCH_SIZE")
        wf, wname, wval = copy_factor(a.cal_write, "WRITE_SIZE")
        fv = read_counter(a.fetch, "FETCH_SIZE")[a.kernel]
        wv = read_counter(a.write, "WRITE_SIZE")[a.kernel]
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        fetch_b, write_b = f_kib * 1024 * ff, w_kib * 1024 * wf
        L += ["Calibration (device copy of exactly 1 GiB):", "",
              f"- FETCH_SIZE read {fval:.0f} KiB for `{fname}`: factor {ff:.4f} bytes per counted byte",
              f"- WRITE_SIZE read {wval:.0f} KiB for `{wname}`: factor {wf:.4f}", "",
              f"`{a.kernel}` per dispatch ({len(fv)} / {len(wv)} dispatches): FETCH_SIZE "
              f"{f_kib:.0f} KiB -> {fetch_b / 1e6:.1f} MB, WRITE_SIZE {w_kib:.0f} KiB -> "
              f"{write_b / 1e6:.1f} MB; HBM traffic {(fetch_b + write_b) / 1e6:.1f} MB per launch.",
              ""]
        if bench and (bench.get("kernels")):
            k = [r for r in bench["kernels"] if r.get("kernel") == a.kernel]
            if k and k[0].get("bytes_per_launch"):
                alg = k[0]["bytes_per_launch"]
                L += [f"Algorithmic bytes per launch (library's count): {alg / 1e6:.1f} MB; "
                      f"measured / algorithmic = {(fetch_b + write_b) / alg:.2f}.", ""]
        rec = dict(kernel=a.kernel, fetch_bytes=round(fetch_b), write_bytes=round(write_b),
                   traffic_bytes=round(fetch_b + write_b), fetch_factor=round(ff, 5),
                   write_factor=round(wf, 5), dispatches=len(fv),
                   sources_sha256=kernel_sources_sha256(a.kernel))
        if bench and isinstance(bench.get("config"), dict):
            rec["workload"] = bench["config"].get("workload")
        L.append("traffic-json: " + json.dumps(rec))
        L.append("")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write("\n".join(L))
    print(a.out)


if __name__ == "__main__":
    sys.exit(main())
