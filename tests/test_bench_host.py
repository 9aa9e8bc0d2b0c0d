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

