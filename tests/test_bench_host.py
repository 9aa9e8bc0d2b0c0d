"""Host-only checks of bench.py's bookkeeping (no GPU)."""

import os
import shutil

import bench


def test_kernel_digest_ignores_comments_but_not_code(tmp_path):
    src = os.path.join(bench.ROOT, "exact_io_aware_11_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    base = bench.kernel_digest("fa_decode.hip", str(dst))
    assert base == bench.kernel_digest("fa_decode.hip", src)
    p = dst / "fa_decode.hip"
    p.write_text("// an added comment line\n" + p.read_text().replace("//", "//   ", 3))
    assert bench.kernel_digest("fa_decode.hip", str(dst)) == base
    # a code change in a shared header invalidates every kernel's record
    h = dst / "fa_common.hpp"
    h.write_text(h.read_text().replace("constexpr float kLn2", "constexpr float kLn2x", 1))
    assert bench.kernel_digest("fa_decode.hip", str(dst)) != base



def test_forward_digest_covers_its_kernel_header(tmp_path):
    src = os.path.join(bench.ROOT, "exact_io_aware_11_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    base = bench.kernel_digest("fa_fwd.hip", str(dst))
    h = dst / "fa_fwd_kernel.hpp"
    h.write_text(h.read_text().replace("constexpr int QK_AHEAD = 6", "constexpr int QK_AHEAD = 5", 1))
    assert bench.kernel_digest("fa_fwd.hip", str(dst)) != base


def test_rate_entry_reports_median_and_best():
    st = {"median_ms": 2.0, "min_ms": 1.6, "calls": 25}
    e = bench.rate_entry(st, 2.0e12, "TFLOP/s", 2516.6, "w")
    assert e["tflops"] == 1000.0 and e["tflops_best"] == 1250.0 and e["calls"] == 25
    assert abs(e["frac"] - 1000.0 / 2516.6) < 1e-4
    g = bench.rate_entry({"median_ms": 1.0, "min_ms": 1.0, "calls": 20}, 8.0e9, "GB/s", 8000.0, "w")
    assert g["GBps"] == 8000.0 and g["frac"] == 1.0


def test_host_info_fields():
    info = bench.host_info()
    assert set(info) == {"cpu_model", "os_cpu_count", "affinity_cores", "blas_threads"}
    assert info["affinity_cores"] >= 1
