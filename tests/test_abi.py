"""C ABI: the library loads, exports what the header declares, and rejects bad
arguments on the host before anything touches a GPU."""
import ctypes
import os
import re

import pytest

import chunked_top_kl_lm_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kd_topk_kl.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kd_\w+)\s*\(", src, flags=re.M)


def test_header_declares_the_entry_points():
    assert set(_declared_functions()) == {"kd_topk_kl_workspace_bytes", "kd_topk_kl_fwd_bwd",
                                          "kd_topk_kl_fwd_bwd_timed", "kd_status_str",
                                          "kd_topk_kl_fwd_workspace_bytes", "kd_topk_kl_bwd_workspace_bytes",
                                          "kd_topk_kl_dw_chunks", "kd_topk_kl_fwd", "kd_topk_kl_bwd",
                                          "kd_topk_cache_workspace_bytes", "kd_topk_cache_build",
                                          "kd_mfma_probe", "kd_topk_kl_fwd_timed", "kd_topk_kl_bwd_timed",
                                          "kd_topk_cache_build_timed", "kd_topk_kl_fwd_bwd_noalloc"}


def test_library_exports_every_declared_symbol():
    L = kd.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code in range(10):
        assert kd.status_str(code) and kd.status_str(code) != "unknown status"
    assert kd.status_str(99) == "unknown status"


def test_workspace_bytes_validation_and_scaling():
    wb = kd.workspace_bytes
    assert wb(0, 8, 8, 1, 1, 0) == 0
    assert wb(8, 0, 8, 1, 1, 0) == 0
    assert wb(8, 8, 8, 9, 1, 0) == 0          # K > V
    assert wb(8, 8, 8, 1, 0, 0) == 0          # chunk < 1
    assert wb(8, 8, 8, 1, 1, 7) == 0          # dtype
    assert wb(8, 8, 5000, 4097, 1, 0) == 0    # K > KD_MAX_K
    # the forward's hit-list strip counts fit 64 KB of LDS up to V = 2096896
    assert wb(64, 64, 2096896, 10, 64, 0) > 0 and wb(64, 64, 2096897, 10, 64, 0) == 0
    assert kd.fwd_workspace_bytes(64, 64, 2096897, 10, 64, 0) == 0
    assert kd.bwd_workspace_bytes(64, 64, 2096897, 10, 64, 0) == 0      # the backward builds them too
    # independent of T beyond the chunk
    a = wb(32768, 2880, 201088, 100, 4096, 0)
    b = wb(262144, 2880, 201088, 100, 4096, 0)
    assert a == b > 0
    # chunk larger than T is T
    assert wb(100, 64, 1000, 10, 5000, 0) == wb(100, 64, 1000, 10, 100, 0)
    # O(chunk*V + V*d): past 8192 rows (one chunk per head-gradient launch)
    # doubling the chunk grows both gradient layouts, 2 * chunk * V * 2 bytes
    c1 = wb(65536, 2880, 201088, 100, 8192, 0)
    c2 = wb(65536, 2880, 201088, 100, 16384, 0)
    assert 0.9 < (c2 - c1) / (2 * 8192 * 201216 * 2) < 1.3
    # below it the transposed layout spans 8192 rows of grouped chunks, so
    # halving the chunk shrinks only the row-major one
    c0 = wb(65536, 2880, 201088, 100, 4096, 0)
    assert 0.9 < (c1 - c0) / (4096 * 201216 * 2) < 1.3
    # fp32 path is larger
    assert wb(512, 256, 4096, 16, 128, 1) > wb(512, 256, 4096, 16, 128, 0)


def test_dw_chunks_grouping():
    dc = kd.dw_chunks
    assert dc(32768, 2880, 201088, 100, 2048, 0) == 4
    assert dc(32768, 2880, 201088, 100, 4096, 0) == 2
    assert dc(32768, 2880, 201088, 100, 8192, 0) == 1
    assert dc(32768, 2880, 201088, 100, 16384, 0) == 1  # at least one
    assert dc(32768, 64, 1000, 10, 1000, 1) == 8        # 1000 rows count as 1024
    assert dc(32768, 64, 1000, 10, 100, 0) == 32        # 100 rows count as 256
    assert dc(3000, 64, 1000, 10, 1024, 0) == 3         # never more chunks than there are
    assert dc(100, 64, 1000, 10, 5000, 0) == 1
    assert dc(0, 64, 1000, 10, 100, 0) == 0             # invalid sizes
    assert dc(100, 64, 1000, 10, 0, 0) == 0


def _call(**kw):
    L = kd.lib()
    args = dict(hidden=0x10000, W=0x20000, dt=0, idx=0x30000, logit=0x40000, mask=None, T=64,
                d=64, V=1000, K=10, tau=1.0, chunk=32, loss=0x50000, gH=0x60000, gW=0x70000,
                rl=None, rk=None, ws=0x100000, wsb=1 << 40, status=None, stream=None)
    args.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kd_topk_kl_fwd_bwd(v(args["hidden"]), v(args["W"]), args["dt"], v(args["idx"]),
                                v(args["logit"]), v(args["mask"]), args["T"], args["d"], args["V"],
                                args["K"], args["tau"], args["chunk"], v(args["loss"]), v(args["gH"]),
                                v(args["gW"]), v(args["rl"]), v(args["rk"]), v(args["ws"]),
                                args["wsb"], v(args["status"]), v(args["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(W=None), 1), (dict(idx=None), 1), (dict(logit=None), 1),
    (dict(loss=None), 1), (dict(gH=None), 1), (dict(gW=None), 1),
    (dict(tau=0.0), 3), (dict(tau=-1.0), 3), (dict(tau=float("nan")), 3), (dict(tau=float("inf")), 3),
    (dict(T=0), 2), (dict(d=0), 2), (dict(V=0), 2), (dict(K=0), 2), (dict(K=1001), 2),
    (dict(chunk=0), 4), (dict(chunk=-5), 4), (dict(dt=3), 5),
    (dict(ws=None), 6), (dict(wsb=1000), 6), (dict(ws=0x100010), 6),
    (dict(hidden=0x10008), 2),
])
def test_host_argument_errors(kw, code):
    # every case fails in host validation, before any HIP call
    assert _call(**kw) == code


def test_timed_entry_requires_events():
    L = kd.lib()
    v = ctypes.c_void_p
    rc = L.kd_topk_kl_fwd_bwd_timed(v(0x10000), v(0x20000), 0, v(0x30000), v(0x40000), None, 64, 64,
                                    1000, 10, 1.0, 32, v(0x50000), v(0x60000), v(0x70000), None, None,
                                    v(0x100000), 1 << 40, None, None, None)
    assert rc == 1


def test_split_workspaces():
    shape = (32768, 2880, 201088, 100, 2048, 0)
    fused, f, b = kd.workspace_bytes(*shape), kd.fwd_workspace_bytes(*shape), kd.bwd_workspace_bytes(*shape)
    # the forward holds no chunk x V gradient buffer; the backward no forward statistics
    assert 0 < f < 64 * 2**20 < b < fused
    assert kd.fwd_workspace_bytes(0, 8, 8, 1, 1, 0) == 0 and kd.bwd_workspace_bytes(8, 8, 8, 9, 1, 0) == 0
    big = (262144, 2880, 201088, 100, 2048, 0)
    assert kd.fwd_workspace_bytes(*big) == f and kd.bwd_workspace_bytes(*big) == b


def _call_fwd(**kw):
    L = kd.lib()
    a = dict(hidden=0x10000, W=0x20000, dt=0, idx=0x30000, logit=0x40000, mask=None, T=64, d=64, V=1000,
             K=10, tau=1.0, chunk=32, loss=0x50000, rl=0x60000, rk=None, ws=0x100000, wsb=1 << 40)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kd_topk_kl_fwd(v(a["hidden"]), v(a["W"]), a["dt"], v(a["idx"]), v(a["logit"]), v(a["mask"]),
                            a["T"], a["d"], a["V"], a["K"], a["tau"], a["chunk"], v(a["loss"]), v(a["rl"]),
                            v(a["rk"]), v(a["ws"]), a["wsb"], None, None)


def _call_bwd(**kw):
    L = kd.lib()
    a = dict(hidden=0x10000, W=0x20000, dt=0, idx=0x30000, logit=0x40000, mask=None, T=64, d=64, V=1000,
             K=10, tau=1.0, chunk=32, rl=0x60000, gl=None, gH=0x70000, ghdt=1, gW=0x80000, acc=0, gWb=None,
             ws=0x100000, wsb=1 << 40)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kd_topk_kl_bwd(v(a["hidden"]), v(a["W"]), a["dt"], v(a["idx"]), v(a["logit"]), v(a["mask"]),
                            a["T"], a["d"], a["V"], a["K"], a["tau"], a["chunk"], v(a["rl"]), v(a["gl"]),
                            v(a["gH"]), a["ghdt"], v(a["gW"]), a["acc"], v(a["gWb"]), v(a["ws"]), a["wsb"],
                            None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(loss=None), 1), (dict(rl=None), 1), (dict(tau=0.0), 3),
    (dict(K=0), 2), (dict(chunk=0), 4), (dict(dt=2), 5), (dict(ws=None), 6), (dict(wsb=10), 6),
])
def test_fwd_host_argument_errors(kw, code):
    assert _call_fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(rl=None), 1), (dict(gH=None, gW=None), 1), (dict(gW=None, gWb=0x90000), 1),
    (dict(ghdt=2), 5), (dict(tau=float("nan")), 3), (dict(V=0), 2), (dict(dt=9), 5), (dict(ws=0x100008), 6),
])
def test_bwd_host_argument_errors(kw, code):
    assert _call_bwd(**kw) == code


def test_topk_cache_host_checks():
    wb = kd.topk_cache_workspace_bytes
    assert wb(0, 8, 8, 1, 1, 0) == 0 and wb(8, 8, 8, 9, 1, 0) == 0 and wb(8, 8, 8, 1, 1, 5) == 0
    a, b = wb(32768, 2880, 201088, 100, 2048, 0), wb(262144, 2880, 201088, 100, 2048, 0)
    # O(chunk * V): the chunk's fp32 logits (2048 x 201216 x 4 bytes) and under 64 MiB more
    z = 2048 * 201216 * 4
    assert a == b > z and a < z + 64 * 2**20



@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(W=None), 1), (dict(idx=None), 1), (dict(logit=None), 1),
    (dict(K=0), 2), (dict(K=1001), 2), (dict(T=0), 2), (dict(chunk=0), 4), (dict(dt=4), 5),
    (dict(ws=None), 6), (dict(wsb=100), 6), (dict(hidden=0x10004), 2),
])
def test_topk_cache_host_argument_errors(kw, code):
    # every case fails in host validation, before any HIP call
    a = dict(hidden=0x10000, W=0x20000, dt=0, T=64, d=64, V=1000, K=10, chunk=32, idx=0x30000, logit=0x40000,
             ws=0x100000, wsb=1 << 40)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    assert kd.lib().kd_topk_cache_build(v(a["hidden"]), v(a["W"]), a["dt"], a["T"], a["d"], a["V"], a["K"],
                                        a["chunk"], v(a["idx"]), v(a["logit"]), v(a["ws"]), a["wsb"], None) == code


def test_mfma_probe_host_errors():
    L = kd.lib()
    assert L.kd_mfma_probe(1, 1, 0, None, None) == 1                          # NULL out
    assert L.kd_mfma_probe(0, 1, 0, ctypes.c_void_p(0x10000), None) == 2     # no blocks
    assert L.kd_mfma_probe(1, 0, 0, ctypes.c_void_p(0x10000), None) == 2     # no iterations


def test_timed_entry_points_require_events():
    L = kd.lib()
    v = ctypes.c_void_p
    p = v(0x10000)
    assert L.kd_topk_kl_fwd_timed(p, p, 0, p, p, None, 64, 64, 1000, 10, 1.0, 32, p, p, None, p, 1 << 40,
                                  None, None, None) == 1
    assert L.kd_topk_kl_bwd_timed(p, p, 0, p, p, None, 64, 64, 1000, 10, 1.0, 32, p, None, p, 1, p, 0, None,
                                  p, 1 << 40, None, None, None) == 1
    assert L.kd_topk_cache_build_timed(p, p, 0, 64, 64, 1000, 10, 32, p, p, p, 1 << 40, None, None) == 1


def test_header_constants_match_the_binding():
    src = open(HEADER).read()
    for name, val in (("KD_NUM_PHASES", kd.KD_NUM_PHASES), ("KD_CACHE_PHASES", kd.KD_CACHE_PHASES),
                      ("KD_BF16", kd.KD_BF16), ("KD_F32", kd.KD_F32)):
        assert re.search(rf"#define {name} (\d+)", src).group(1) == str(val), name
    assert len(kd.PHASES) == kd.KD_NUM_PHASES and len(kd.CACHE_PHASES) == kd.KD_CACHE_PHASES


def _call_noalloc(**kw):
    L = kd.lib()
    a = dict(hidden=0x10000, W=0x20000, dt=0, idx=0x30000, logit=0x40000, mask=None, T=64, d=64, V=1000,
             K=10, tau=1.0, chunk=32, loss=0x50000, gH=0x60000, gW=0x70000, rl=None, rk=None, status=None)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kd_topk_kl_fwd_bwd_noalloc(v(a["hidden"]), v(a["W"]), a["dt"], v(a["idx"]), v(a["logit"]),
                                        v(a["mask"]), a["T"], a["d"], a["V"], a["K"], a["tau"], a["chunk"],
                                        v(a["loss"]), v(a["gH"]), v(a["gW"]), v(a["rl"]), v(a["rk"]),
                                        v(a["status"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(gW=None), 1), (dict(tau=0.0), 3), (dict(K=0), 2), (dict(chunk=0), 4),
    (dict(dt=3), 5),
    # the 32K workload's head needs ~2.8 GB of workspace even with one chunk
    # per head-gradient launch: refused before any device call
    (dict(T=32768, d=2880, V=201088, K=100, chunk=2048), 9),
    (dict(T=64, d=4096, V=100000, K=100, chunk=64), 9),
])
def test_noalloc_host_errors(kw, code):
    assert _call_noalloc(**kw) == code
