"""The host-side launch plan (csrc/plan.cpp: validation, GEMM-form choices,
workspace layouts) built on its own with g++ under the address and
undefined-behaviour sanitizers, driven over a sweep of shapes that includes
the library's limits and rejected shapes; every answer must equal what the
library returns through the C ABI, and no sanitizer may report."""
import os
import shutil
import subprocess

import pytest

import sparse_mixture_experts_scan_amd as moe
from sparse_mixture_experts_scan_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_scan_amd", "csrc")

FIELDS = ("topk_idx", "topk_w", "block_counts", "counts", "offsets", "num_tiles",
          "tile_expert", "row_token", "tok_row", "row_w", "xs", "h", "y", "y_parts", "down_sched",
          "block_probs", "norm_rs", "xn", "router_partial", "wdeq", "total")


def shapes():
    out = []
    for T in (0, 1, 16, 31, 32, 33, 1000, 4096, 8192, 1 << 24, (1 << 24) + 1):
        for (d, f, E, k) in ((4096, 14336, 8, 2), (4096, 3584, 64, 8), (128, 512, 8, 2),
                             (64, 64, 1, 1), (192, 320, 6, 3), (32768, 131072, 64, 8),
                             (100, 512, 8, 2), (256, 512, 65, 2), (256, 512, 8, 9),
                             (256, 512, 4, 5), (32832, 512, 8, 2)):
            for dtype in (0, 1, 2):
                for block in (0, 1):
                    out.append((T, d, f, E, k, dtype, block))
    return out


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_plan_under_sanitizers_matches_library(driver):
    sh = shapes()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], input="".join(" ".join(map(str, s)) + "\n" for s in sh),
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert len(lines) == len(sh)
    n_ok = 0
    for s, line in zip(sh, lines):
        T, d, f, E, k, dtype, block = s
        vals = [int(v) for v in line.split()]
        if block and dtype == B.MOE_W4A16:
            assert moe.moe_block_workspace_size(T, d, f, E, k, dtype) == 0
            continue
        size = (moe.moe_block_workspace_size if block else moe.moe_ffn_workspace_size)(
            T, d, f, E, k, dtype)
        if vals[0] != 0:
            assert size == 0, s
            continue
        n_ok += 1
        lay = (moe.moe_block_workspace_layout if block else moe.moe_ffn_workspace_layout)(
            T, d, f, E, k, dtype)
        head = [lay.block_rows, lay.max_rows, lay.router_blocks, lay.y_part_rows,
                lay.gemm_variant, lay.down_splits, lay.tokens_in_place, lay.y_weighted]
        assert vals[1:9] == head, s
        assert vals[9:9 + len(FIELDS)] == [getattr(lay, n) for n in FIELDS], s
        assert size == lay.total
        assert vals[-1] == moe.moe_ffn_backward_workspace_size(T, d, f, E, k), s
    assert n_ok > 100
