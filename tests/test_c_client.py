"""The C ABI from C: tests/c_abi_client.c is compiled as C99 against
include/kd_topk_kl.h, linked against the built library and run (host-side
entry points only, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunked_top_kl_lm_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client_compiles_links_and_runs(tmp_path):
    import chunked_top_kl_lm_amd as kd
    kd.lib()                                  # the library is built and loads
    exe = tmp_path / "c_abi_client"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"),
           "-L", PKG, "-lkdtopk", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = dict(l.split(" ", 1) for l in out.stdout.strip().splitlines())
    assert lines["null_args"].startswith("1 ")
    assert lines["bad_shape_size"] == "0"
    ws = int(lines["workspace"].split()[0])
    assert ws == kd.workspace_bytes(32768, 2880, 201088, 100, 2048, kd.KD_BF16)
    assert lines["workspace"].endswith("same_for_256k 1")
