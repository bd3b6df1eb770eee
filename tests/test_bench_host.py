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


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
