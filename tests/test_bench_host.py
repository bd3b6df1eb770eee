"""Host-side pieces of the measurement: kernel-name normalisation, the
source hash that keeps stale counter summaries out of the bench line, and
the one-GPU contract of bench.py."""
import os
import subprocess
import sys

import rocprof_summary as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_short_name():
    assert R.short_name("void gk::k_gemm_mfma<128, 128, true, true, 4>(long, long, long, "
                        "unsigned short const*, long)") == "k_gemm_mfma<128, 128, true, true, 4>"
    assert R.short_name("gk::k_attn_bwd_dkv(unsigned short const*, int)") == "k_attn_bwd_dkv"
    assert R.short_name("void at::native::vectorized_elementwise_kernel<4, at::native::"
                        "FillFunctor<float>, std::array<char*, 1ul> >(int, at::native::"
                        "FillFunctor<float>, std::array<char*, 1ul>)").startswith(
        "at::native::vectorized_elementwise_kernel<4,")


def test_source_hash_depends_on_defining_file():
    a = R.kernel_sources_sha256("k_gemm_mfma<128, 128, true, true, 4>")
    b = R.kernel_sources_sha256("k_gemm_mfma_db<false, false, 2>")
    c = R.kernel_sources_sha256("k_attn_bwd_dkv")
    assert a == R.kernel_sources_sha256("k_gemm_mfma<256, 128, false, false, 1>")
    assert a == b          # both defined in the GEMM source
    assert a != c


def test_load_traffic_unknown_kernel_is_none():
    assert R.load_traffic("k_no_such_kernel") is None


def test_load_traffic_matches_workload(tmp_path, monkeypatch):
    """A summary's traffic is reported only for the workload it was taken
    on: the same kernel on another model shape gets none."""
    k = "k_gemm_dma<256, 256, true, true, 4>"
    rec = {"kernel": k, "traffic_bytes": 123, "sources_sha256": R.kernel_sources_sha256(k),
           "workload": "shape A"}
    (tmp_path / "p.md").write_text("# t\n\ntraffic-json: " + __import__("json").dumps(rec) + "\n")
    monkeypatch.setattr(R, "PROFILES", str(tmp_path))
    assert R.load_traffic(k, "shape A")["traffic_bytes"] == 123
    assert R.load_traffic(k, "shape B") is None
    assert R.load_traffic(k)["traffic_bytes"] == 123
    rec["sources_sha256"] = "0" * 64                   # sources changed since
    (tmp_path / "p.md").write_text("traffic-json: " + __import__("json").dumps(rec) + "\n")
    assert R.load_traffic(k, "shape A") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_clock_parsing_and_host_info():
    sys.path.insert(0, ROOT)
    import bench
    txt = "0: 500Mhz\n1: 1900Mhz\n2: 2400Mhz *\n"
    assert bench.parse_sclk(txt) == 2400
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz\n") is None
    info = bench.host_cpu_info()
    assert info["cores"] >= 1 and "blas_threads" in info


def test_counter_table_takes_one_step_between_markers(tmp_path):
    """--table counts the dispatches from the marker kernel's second launch
    up to its third (one timed step), one value per dispatch and counter,
    averaged per kernel."""
    import csv
    d = tmp_path / "run"
    d.mkdir()
    seq = [("k_embed", 1.0), ("k_a", 10.0), ("k_b", 5.0),      # warm-up step
           ("k_embed", 2.0), ("k_a", 20.0), ("k_a", 40.0), ("k_b", 7.0),   # timed step
           ("k_embed", 3.0), ("k_a", 99.0)]                   # next step
    with open(d / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(seq, start=1):
            name = f"void gk::{k}(int)"
            w.writerow([i, name, "MfmaUtil", v])
            w.writerow([i, name, "FETCH_SIZE", 2 * v])
    steps = R.read_dispatches(str(d), "k_embed")
    assert [n for n, _ in steps] == ["k_embed", "k_a", "k_a", "k_b"]
    assert R.per_kernel_mean(steps, "MfmaUtil") == {"k_embed": 2.0, "k_a": 30.0, "k_b": 7.0}
    assert R.per_kernel_mean(steps, "FETCH_SIZE")["k_a"] == 60.0
    assert len(R.read_dispatches(str(d), None)) == len(seq)
