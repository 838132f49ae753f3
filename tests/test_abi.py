"""The C-ABI library: it loads, exports every function the header declares, and
rejects bad arguments with the documented codes before touching a GPU."""
import ctypes
import os
import re

import pytest

import sparse_gather_mla_amd as sgm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_gather_decode.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_gather_decode_\w+)\s*\(", src)))


def _codes():
    src = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(MLA_GD_\w+)\s+(\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sgm.LIB_PATH):
        pytest.fail("library not built (run sparse_gather_mla_amd/build.py)")
    return sgm.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) == 13, names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strerror(lib):
    c = _codes()
    assert lib.mla_gather_decode_abi_version() == c["MLA_GD_ABI_VERSION"]
    seen = set()
    for name in ("MLA_GD_OK", "MLA_GD_E_INVAL", "MLA_GD_E_ALIGN", "MLA_GD_E_WORKSPACE", "MLA_GD_E_UNSUPPORTED",
                 "MLA_GD_E_HIP", "MLA_GD_E_DEVICE_CHECK"):
        s = lib.mla_gather_decode_strerror(c[name]).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.mla_gather_decode_strerror(12345).decode() == "unknown error"


def _dims(**kw):
    base = dict(hidden=256, q_lora_rank=64, kv_lora_rank=64, qk_nope_head_dim=32, qk_rope_head_dim=16,
                v_head_dim=32, n_heads=4, block_size=16, max_blocks_per_seq=8, n_blocks=16, n_prior=32,
                max_tokens=2, softmax_scale=0.144, norm_eps=1e-6, flags=0)
    base.update(kw)
    return sgm._Dims(**base)


def _create(lib, d):
    h = ctypes.c_void_p()
    rc = lib.mla_gather_decode_create(ctypes.byref(d), 0, ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    ({}, "MLA_GD_OK"),
    ({"hidden": 0}, "MLA_GD_E_INVAL"),
    ({"n_prior": -1}, "MLA_GD_E_INVAL"),
    ({"qk_rope_head_dim": 15}, "MLA_GD_E_INVAL"),
    ({"flags": 16}, "MLA_GD_E_INVAL"),
    ({"flags": 1 | 8}, "MLA_GD_E_INVAL"),  # fused and single launch together
    ({"norm_eps": -1.0}, "MLA_GD_E_INVAL"),
    ({"softmax_scale": float("nan")}, "MLA_GD_E_INVAL"),
    ({"hidden": 260}, "MLA_GD_E_UNSUPPORTED"),
    ({"kv_lora_rank": 1024}, "MLA_GD_E_UNSUPPORTED"),
    ({"kv_lora_rank": 72}, "MLA_GD_E_UNSUPPORTED"),
    ({"qk_rope_head_dim": 256}, "MLA_GD_E_UNSUPPORTED"),
    ({"qk_rope_head_dim": 72, "kv_lora_rank": 64}, "MLA_GD_E_UNSUPPORTED"),
    ({"kv_lora_rank": 96}, "MLA_GD_E_UNSUPPORTED"),
    ({"max_tokens": 5000}, "MLA_GD_E_UNSUPPORTED"),
    ({"q_lora_rank": 16384}, "MLA_GD_E_UNSUPPORTED"),
    ({"n_prior": 262144 + 1}, "MLA_GD_E_UNSUPPORTED"),
    # more than 64 heads: at most 64 core splits of 2560 row ids
    ({"n_heads": 72, "n_prior": 163840}, "MLA_GD_OK"),
    ({"n_heads": 72, "n_prior": 163840 + 1}, "MLA_GD_E_UNSUPPORTED"),
    ({"n_heads": 64, "n_prior": 163840 + 1}, "MLA_GD_OK"),
])
def test_create_validates_dims(lib, kw, code):
    rc, h = _create(lib, _dims(**kw))
    assert rc == _codes()[code]
    if rc == 0:
        assert h.value
        lib.mla_gather_decode_destroy(h)
    else:
        assert not h.value


def test_workspace_size_and_step_argument_checks(lib):
    c = _codes()
    rc, h = _create(lib, _dims(max_tokens=4))
    assert rc == 0
    try:
        assert lib.mla_gather_decode_workspace_size(h, 0) == 0
        assert lib.mla_gather_decode_workspace_size(h, 5) == 0
        sizes = [lib.mla_gather_decode_workspace_size(h, t) for t in (1, 2, 3, 4)]
        assert all(s > 0 and s % 256 == 0 for s in sizes)
        assert sizes == sorted(sizes)  # a workspace for n tokens serves every smaller step
        assert lib.mla_gather_decode_workspace_size(None, 1) == 0
        tn = sgm._Tensors()
        # missing tensors / workspace / handle: rejected before any device work
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ctypes.c_void_p(256), 1 << 20, None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_step(None, ctypes.byref(tn), 1, ctypes.c_void_p(256), 1 << 20, None) == c["MLA_GD_E_INVAL"]
        for f in sgm.TENSOR_FIELDS:
            if f != "gather_rows_out":
                setattr(tn, f, 4096)
        ws = ctypes.c_void_p(1 << 20)
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 0, ws, sizes[0], None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 5, ws, sizes[0], None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ws, sizes[0] - 1, None) == c["MLA_GD_E_WORKSPACE"]
        tn.wq_b = 4096 + 8  # bf16 pointers need 16-byte alignment
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ws, sizes[0], None) == c["MLA_GD_E_ALIGN"]
        tn.wq_b = 4096
        tn.positions = 4096 + 2
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ws, sizes[0], None) == c["MLA_GD_E_ALIGN"]
        tn.positions = 4096
        tn.token_seq = 4096 + 2  # optional, but 4-byte aligned when given
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ws, sizes[0], None) == c["MLA_GD_E_ALIGN"]
        tn.token_seq = None
        assert lib.mla_gather_decode_step(h, ctypes.byref(tn), 1, ctypes.c_void_p((1 << 20) + 16), sizes[0],
                                          None) == c["MLA_GD_E_ALIGN"]
        assert lib.mla_gather_decode_workspace_init(h, None, 1024, None) == c["MLA_GD_E_INVAL"]
        for T in (1, 4):
            n = lib.mla_gather_decode_kernel_count(h, T)
            assert n >= 1
            names = [lib.mla_gather_decode_kernel_name(h, T, i).decode() for i in range(n)]
            assert all(names) and len(set(names)) == len(names)
            assert "k_core" in names and names[-1] == ("k_oproj" if T <= 3 else "k_out")
            assert lib.mla_gather_decode_kernel_name(h, T, n) == b""
        assert lib.mla_gather_decode_kernel_count(h, 0) == 0
        assert lib.mla_gather_decode_kernel_count(h, 5) == 0
        assert lib.mla_gather_decode_kernel_name(h, 0, 0) == b""
        # profiled step: a missing or short event list is rejected
        assert lib.mla_gather_decode_step_profiled(h, ctypes.byref(tn), 1, ws, sizes[0], None, None, 0) == c["MLA_GD_E_INVAL"]
        ev = (ctypes.c_void_p * 2)(1, 1)
        assert lib.mla_gather_decode_step_profiled(h, ctypes.byref(tn), 1, ws, sizes[0], None, ev, 2) == c["MLA_GD_E_INVAL"]
    finally:
        lib.mla_gather_decode_destroy(h)
    lib.mla_gather_decode_destroy(None)  # NULL-safe


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(sgm, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        sgm.load_library(str(tmp_path / "missing.so"))


def test_kernel_lists_of_both_paths(lib):
    """Steps of up to 3 tokens run the GEMV path; larger ones the matrix-core
    path with its two extra kernels.  The workspace covers both."""
    rc, h = _create(lib, _dims(max_tokens=40))
    assert rc == 0
    try:
        def names(T):
            n = lib.mla_gather_decode_kernel_count(h, T)
            return [lib.mla_gather_decode_kernel_name(h, T, i).decode() for i in range(n)]
        gemv = names(3)
        mfma = names(4)
        # the GEMV path's o-projection writes the output itself (no k_out)
        assert gemv == ["k_down", "k_qup", "k_absorb", "k_core", "k_oabsorb", "k_oproj"]
        full = ["k_prep", "k_down", "k_qa", "k_qup", "k_absorb", "k_core", "k_oabsorb", "k_oproj", "k_out"]
        # the output absorption combines the core's splits itself
        assert mfma == full and names(40) == full
        sizes = [lib.mla_gather_decode_workspace_size(h, t) for t in range(1, 41)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    finally:
        lib.mla_gather_decode_destroy(h)



def test_fused_flag_kernel_list(lib):
    """The fused variant replaces k_absorb + k_core by one launch on the GEMV
    path (up to 16 heads); more heads, or steps on the matrix-core path, keep
    the separate kernels."""
    c = _codes()

    def names(h, T):
        n = lib.mla_gather_decode_kernel_count(h, T)
        return [lib.mla_gather_decode_kernel_name(h, T, i).decode() for i in range(n)]

    rc, h = _create(lib, _dims(max_tokens=12, flags=c["MLA_GD_FLAG_FUSED"]))
    assert rc == 0
    try:
        assert names(h, 1) == ["k_down", "k_qup", "k_absorb_core", "k_oabsorb", "k_oproj"]
        assert names(h, 3) == names(h, 1)
        assert "k_absorb_core" not in names(h, 4) and "k_core" in names(h, 4)
        # the counters live in the workspace, so fused and separate sizes agree
        rc2, h2 = _create(lib, _dims(max_tokens=12))
        assert rc2 == 0
        try:
            assert lib.mla_gather_decode_workspace_size(h, 12) == lib.mla_gather_decode_workspace_size(h2, 12)
        finally:
            lib.mla_gather_decode_destroy(h2)
    finally:
        lib.mla_gather_decode_destroy(h)
    rc, h = _create(lib, _dims(n_heads=20, flags=c["MLA_GD_FLAG_FUSED"]))
    assert rc == 0
    try:
        assert "k_core" in names(h, 1) and "k_absorb_core" not in names(h, 1)
    finally:
        lib.mla_gather_decode_destroy(h)


def test_single_launch_flag_kernel_list(lib):
    """The single-launch variant runs the whole step as one kernel on the GEMV
    path (up to 3 tokens, up to 16 heads); larger steps, more heads or more
    prior positions than its splits hold keep the separate kernels."""
    c = _codes()

    def names(h, T):
        n = lib.mla_gather_decode_kernel_count(h, T)
        return [lib.mla_gather_decode_kernel_name(h, T, i).decode() for i in range(n)]

    rc, h = _create(lib, _dims(max_tokens=12, flags=c["MLA_GD_FLAG_SINGLE_LAUNCH"]))
    assert rc == 0
    try:
        assert names(h, 1) == ["k_step"] and names(h, 3) == ["k_step"]
        assert names(h, 4)[0] == "k_prep" and "k_step" not in names(h, 4)
        sizes = [lib.mla_gather_decode_workspace_size(h, t) for t in range(1, 13)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    finally:
        lib.mla_gather_decode_destroy(h)
    for kw in ({"n_heads": 20}, {"n_prior": 64 * 2048 + 32, "max_blocks_per_seq": 8300, "n_blocks": 16600}):
        rc, h = _create(lib, _dims(flags=c["MLA_GD_FLAG_SINGLE_LAUNCH"], **kw))
        assert rc == 0, kw
        try:
            assert names(h, 1)[0] == "k_down", kw
        finally:
            lib.mla_gather_decode_destroy(h)


def test_debug_checks_flag_and_status_arguments(lib):
    """The debug-checks flag is accepted; the status query rejects a handle
    created without it and null arguments before any GPU call."""
    c = _codes()
    rc, h = _create(lib, _dims(flags=c["MLA_GD_FLAG_DEBUG_CHECKS"]))
    assert rc == 0
    bits = ctypes.c_uint32(0)
    try:
        assert lib.mla_gather_decode_debug_status(h, None, ctypes.byref(bits), None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_debug_status(h, ctypes.c_void_p(4096), None, None) == c["MLA_GD_E_INVAL"]
    finally:
        lib.mla_gather_decode_destroy(h)
    rc, h = _create(lib, _dims())
    assert rc == 0
    try:
        assert lib.mla_gather_decode_debug_status(h, ctypes.c_void_p(4096), ctypes.byref(bits), None) == c["MLA_GD_E_INVAL"]
    finally:
        lib.mla_gather_decode_destroy(h)
    assert lib.mla_gather_decode_debug_status(None, ctypes.c_void_p(4096), ctypes.byref(bits), None) == c["MLA_GD_E_INVAL"]
    # distinct check bits
    bits_def = [c[k] for k in ("MLA_GD_CHECK_SLOT_RANGE", "MLA_GD_CHECK_BLOCK_RANGE", "MLA_GD_CHECK_TABLE_COLUMN",
                               "MLA_GD_CHECK_SLOT_SHARED", "MLA_GD_CHECK_SEQ_RANGE")]
    assert sorted(bits_def) == [1, 2, 4, 8, 16]


def test_binding_constants_match_the_header():
    c = _codes()
    for k in ("MLA_GD_FLAG_FUSED", "MLA_GD_FLAG_GRAPH", "MLA_GD_FLAG_DEBUG_CHECKS", "MLA_GD_CHECK_SLOT_RANGE",
              "MLA_GD_CHECK_BLOCK_RANGE", "MLA_GD_CHECK_TABLE_COLUMN", "MLA_GD_CHECK_SLOT_SHARED",
              "MLA_GD_CHECK_SEQ_RANGE"):
        assert getattr(sgm, k) == c[k], k


def test_noalloc_step_rejections_before_any_device_work(lib):
    """The allocation-free step rejects a null handle or tensors, a handle with
    debug checks, an out-of-range token count, and a step whose workspace would
    exceed the static scratch (128 heads of the DeepSeek-V3.2 dims), all before
    it touches a GPU."""
    c = _codes()
    tn = sgm._Tensors()
    assert lib.mla_gather_decode_step_noalloc(None, ctypes.byref(tn), 1, None) == c["MLA_GD_E_INVAL"]
    rc, h = _create(lib, _dims(flags=c["MLA_GD_FLAG_DEBUG_CHECKS"]))
    assert rc == 0
    try:
        assert lib.mla_gather_decode_step_noalloc(h, ctypes.byref(tn), 1, None) == c["MLA_GD_E_INVAL"]
    finally:
        lib.mla_gather_decode_destroy(h)
    rc, h = _create(lib, _dims(max_tokens=2))
    assert rc == 0
    try:
        assert lib.mla_gather_decode_step_noalloc(h, None, 1, None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_step_noalloc(h, ctypes.byref(tn), 0, None) == c["MLA_GD_E_INVAL"]
        assert lib.mla_gather_decode_step_noalloc(h, ctypes.byref(tn), 3, None) == c["MLA_GD_E_INVAL"]
    finally:
        lib.mla_gather_decode_destroy(h)
    big = _dims(hidden=7168, q_lora_rank=1536, kv_lora_rank=512, qk_nope_head_dim=128, qk_rope_head_dim=64,
                v_head_dim=128, n_heads=128, block_size=64, max_blocks_per_seq=2048, n_blocks=262144,
                n_prior=2048, max_tokens=128)
    rc, h = _create(lib, big)
    assert rc == 0
    try:
        limit = 32 << 20
        assert lib.mla_gather_decode_workspace_size(h, 128) > limit
        assert lib.mla_gather_decode_step_noalloc(h, ctypes.byref(tn), 128, None) == c["MLA_GD_E_WORKSPACE"]
    finally:
        lib.mla_gather_decode_destroy(h)
    src = open(HEADER).read()
    assert "#define MLA_GD_STATIC_SCRATCH_BYTES (32u << 20)" in src


def test_plan_log_prints_each_step_size_once():
    """MLA_GD_LOG set at create: the first step of each size prints its work
    decomposition to stderr (here steps rejected for a short workspace, after
    planning and before any device work)."""
    import subprocess
    import sys
    import textwrap

    code = textwrap.dedent("""
        import ctypes
        import sparse_gather_mla_amd as sgm
        from tests.test_abi import _codes, _dims
        lib = sgm.load_library()
        h = ctypes.c_void_p()
        d = _dims(max_tokens=8, n_heads=72, kv_lora_rank=128)
        assert lib.mla_gather_decode_create(ctypes.byref(d), 0, ctypes.byref(h)) == 0
        tn = sgm._Tensors()
        for f in sgm.TENSOR_FIELDS:
            if f != "gather_rows_out":
                setattr(tn, f, 4096)
        ws = ctypes.c_void_p(1 << 20)
        for T in (1, 5, 1, 5):
            assert lib.mla_gather_decode_step(h, ctypes.byref(tn), T, ws, 256, None) == _codes()["MLA_GD_E_WORKSPACE"]
        lib.mla_gather_decode_destroy(h)
    """)
    import os

    env = dict(os.environ, MLA_GD_LOG="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[mla_gd] T=")]
    assert len(lines) == 2, r.stderr
    assert lines[0].startswith("[mla_gd] T=1: GEMV path") and "one 16-head tile per wave" in lines[0]
    assert lines[1].startswith("[mla_gd] T=5: matrix-core path")
