"""CPU checks of the kernels' address arithmetic and of the workspace carve-up.

tests/index_check.cpp includes the library's own kd_layout.hpp (the index
functions the GEMM epilogues, hit lists and operand staging call on the
device) and kd_plan.hpp (the plan and workspace offsets), and is built here
with the host compiler under the address and undefined-behaviour
sanitizers.  Over swept ragged shapes it checks that every access stays in
its buffer and reaches its own element, and that the plan's buffers are
aligned, disjoint, inside the workspace and as large as the kernels index
them (see the file's header).  Each planted mistake -- a head-gradient
resource sized to the padded tile instead of the vocabulary, a lost column
guard, the gradient staging without its swizzle, one G^T slot for a group
of chunks, a workspace total that leaves out the last buffer, the cache
builder's logit rows at the unpadded vocabulary stride -- must fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "index_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("index_check") / "index_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "chunked_top_kl_lm_amd", "csrc"), "-I", os.path.join(ROOT, "include"), SRC,
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)


def test_every_access_in_bounds_and_plan_consistent(checker):
    r = _run(checker)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "failures: 0" in r.stdout
    n = int(r.stdout.split("index checks: ")[1].split(",")[0])
    assert n > 10_000_000


@pytest.mark.parametrize("plant,sign", [
    ("accum-row-guard", "element past the matrix lands inside"),
    ("accum-col-guard", "element past the matrix lands inside"),
    ("g-stage-swizzle", "G read"),
    ("gt-group-stride", "G^T slot"),
    ("plan-total", "heap-buffer-overflow"),
    ("cache-z-stride", "logit store"),
])
def test_planted_mistakes_are_caught(checker, plant, sign):
    r = _run(checker, "--plant", plant)
    assert r.returncode != 0
    assert sign in r.stdout + r.stderr
