"""The allocation-free entry point (mla_gather_decode_step_noalloc), through
the C ABI, against the workspace entry point (mla_gather_decode_step) on the
same inputs: two calls in a row, the second with fewer tokens, so the static
scratch holds the first call's contents when the second one runs.  The two
entry points run the same kernels with the same plan, so outputs, written
cache rows and resolved rows must agree bit for bit."""
import sys

import pytest
import torch

from sparse_gather_mla_amd import Dims, MlaGatherDecode
from tests.harness import bf16_to_f64, oracle_reference, token_slice, within_tol
from workload import config_by_name, make_inputs, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(mod, g, T, P):
    """One step through each entry point on identical copies of the pool."""
    pool0 = g["kv_cache"].clone()
    rows_ws = torch.full((T, P), -7, dtype=torch.int32, device="cuda")
    out_ws = mod(g, gather_rows_out=rows_ws).clone()
    pool_ws = g["kv_cache"].clone()
    g["kv_cache"].copy_(pool0)
    rows_na = torch.full((T, P), -7, dtype=torch.int32, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    mod(g, out=out_na, gather_rows_out=rows_na, noalloc=True)
    torch.cuda.synchronize()
    return (out_ws, rows_ws, pool_ws), (out_na, rows_na, g["kv_cache"].clone())


@pytest.mark.parametrize("name,first,second", [("batch32", 32, 5), ("ds32_slice", 1, 1)])
def test_noalloc_matches_workspace_entry_point(name, first, second):
    wl = config_by_name(name)
    sh = wl.shape
    _say(f"[noalloc] {name}: {first} then {second} tokens")
    inp = make_inputs(wl, with_pool=False)
    g_all = to_device(wl, inp, device="cuda")
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    for step, T in enumerate((first, second)):
        toks = list(range(T)) if step == 0 else list(range(sh.n_tokens - T, sh.n_tokens))
        g = token_slice(g_all, toks)
        g["kv_cache"] = g_all["kv_cache"]
        (o1, r1, p1), (o2, r2, p2) = _both(mod, g, T, sh.n_prior)
        assert torch.equal(r1, r2), "resolved rows differ"
        assert torch.equal(o1, o2), "outputs differ"
        assert torch.equal(p1, p2), "cache pools differ"
        ref = oracle_reference(wl, inp, toks)
        ok, err, bound = within_tol(bf16_to_f64(o2), ref["out"])
        _say(f"[noalloc] {name} call {step + 1} ({T} tokens): bit-equal; vs oracle max err {err:.3e} bound {bound:.3e}")
        assert ok


def test_noalloc_rejects_steps_beyond_the_static_scratch():
    wl = config_by_name("fullhead64")
    sh = wl.shape
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens, allocate_workspace=False)
    assert mod.workspace_size(sh.n_tokens) > (32 << 20)
    inp = make_inputs(wl.with_tokens(64), with_pool=False)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    g["kv_cache"] = torch.empty((sh.n_blocks, 1, sh.block_size, sh.kv_row_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="workspace too small"):
        mod(g, noalloc=True)
