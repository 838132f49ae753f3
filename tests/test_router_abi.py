"""Host-side checks of the router top-K C ABI: exports, limits and argument errors (no GPU work)."""
import ctypes
import os
import re

import pytest

import sparse_gather_mla_amd as sgm
from sparse_gather_mla_amd import router

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rmsnorm_router_topk.h")


def _codes():
    return {k: int(v) for k, v in re.findall(r"#define\s+(RT_\w+)\s+(\d+)", open(HEADER).read())}


def test_router_symbols_exported():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(rmsnorm_router_topk\w*)\s*\(", src)))
    assert names == ["rmsnorm_router_topk", "rmsnorm_router_topk_typed", "rmsnorm_router_topk_workspace_size"]
    lib = sgm.load_library()
    for n in names:
        assert hasattr(lib, n)


def test_router_workspace_limits():
    assert router.workspace_size(1, 7168, 256) > 0
    assert router.workspace_size(128, 7168, 256) > 0
    for bad in ((0, 7168, 256), (129, 7168, 256), (1, 7100, 256), (1, 7168, 252), (1, 7168, 2048)):
        assert router.workspace_size(*bad) == 0, bad


def test_router_argument_errors_before_any_launch():
    c = _codes()
    lib = router._lib()
    p = ctypes.c_void_p(4096)  # never dereferenced: every case fails validation first
    ip = ctypes.c_void_p(4096)

    def call(T=1, H=256, E=16, K=2, eps=1e-6, act=0, ws=1 << 20, hs=p, w=p):
        return lib.rmsnorm_router_topk(hs, p, w, None, T, H, E, K, eps, act, p, ip, p, p, ws, None)

    assert call(hs=None) == c["RT_E_INVAL"]
    assert call(T=0) == c["RT_E_INVAL"]
    assert call(T=200) == c["RT_E_UNSUPPORTED"]
    assert call(H=200) == c["RT_E_UNSUPPORTED"]
    assert call(K=0) == c["RT_E_INVAL"]
    assert call(K=17) == c["RT_E_INVAL"]  # more than n_experts
    assert call(act=2) == c["RT_E_INVAL"]
    assert call(eps=-1.0) == c["RT_E_INVAL"]
    assert call(w=ctypes.c_void_p(4098)) == c["RT_E_ALIGN"]
    assert call(ws=16) == c["RT_E_WORKSPACE"]


def test_router_typed_entry_rejects_unknown_dtype_first():
    c = _codes()
    lib = router._lib()
    p = ctypes.c_void_p(4096)
    for dt in (2, -1):
        assert lib.rmsnorm_router_topk_typed(dt, p, p, p, None, 1, 256, 16, 2, 1e-6, 0, p, p, p, p, 1 << 20,
                                             None) == c["RT_E_INVAL"]
    # a known dtype reaches the ordinary checks
    assert lib.rmsnorm_router_topk_typed(c["RT_DTYPE_FP16"], p, p, p, None, 0, 256, 16, 2, 1e-6, 0, p, p, p, p,
                                         1 << 20, None) == c["RT_E_INVAL"]
