"""Guard blocks around every buffer the step writes, on the GPU, through the C ABI.

The parity tests compare the whole cache pool with its copy, so a stray write
inside the pool is caught there; these tests catch writes outside the caller's
buffers.  The pool, the output, the gathered-row output and the workspace each
sit in the middle of a larger allocation whose head and tail hold a fixed
pattern.  After a step every guard must still hold the pattern, and the
results must be bit-identical to the same step on plain, unguarded buffers.
Three shapes: the GEMV path (one token, 16 heads), the matrix-core path
(8 tokens, 16 heads) and the 128-head core (8 tokens, 128 heads).
"""
import sys

import pytest
import torch

from sparse_gather_mla_amd import Dims, MlaGatherDecode
from tests.harness import gpu_inputs
from workload import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

GUARD = 1 << 16  # bytes of guard on each side (a multiple of 256 keeps the payload aligned)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _guarded(nbytes, device="cuda"):
    """A byte buffer with GUARD bytes of pattern on each side; returns (whole, payload)."""
    whole = torch.empty(GUARD + nbytes + GUARD, dtype=torch.uint8, device=device)
    pat = (torch.arange(whole.numel(), device=device) * 37 + 11).to(torch.uint8)
    whole.copy_(pat)
    return whole, whole[GUARD:GUARD + nbytes]


def _guards_intact(whole, nbytes):
    pat = (torch.arange(whole.numel(), device=whole.device) * 37 + 11).to(torch.uint8)
    head_ok = torch.equal(whole[:GUARD], pat[:GUARD])
    tail_ok = torch.equal(whole[GUARD + nbytes:], pat[GUARD + nbytes:])
    return head_ok and tail_ok


CASES = [
    ("ds32_slice", 1),
    ("batch32", 8),
    ("fullhead64", 8),
]


@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}_T{t}" for n, t in CASES])
def test_no_write_outside_the_callers_buffers(name, T):
    wl = next(c for c in CONFIGS if c.name == name).with_tokens(T)
    sh = wl.shape
    _say(f"[guards] {name} T={T} nh={sh.n_heads}")
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=T)

    # reference: the same step on plain buffers
    pool_ref = g["kv_cache"].clone()
    ref_in = dict(g, kv_cache=pool_ref)
    out_ref = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device="cuda")
    rows_ref = torch.empty((T, sh.n_prior), dtype=torch.int32, device="cuda")
    mod(ref_in, out=out_ref, gather_rows_out=rows_ref)
    torch.cuda.synchronize()

    # guarded copies of the pool, the output, the row output and the workspace
    pool_bytes = g["kv_cache"].numel() * 2
    pool_whole, pool_pay = _guarded(pool_bytes)
    pool_g = pool_pay.view(torch.bfloat16).view(g["kv_cache"].shape)
    pool_g.copy_(g["kv_cache"])
    out_whole, out_pay = _guarded(T * sh.hidden * 2)
    out_g = out_pay.view(torch.bfloat16).view(T, sh.hidden)
    rows_whole, rows_pay = _guarded(T * sh.n_prior * 4)
    rows_g = rows_pay.view(torch.int32).view(T, sh.n_prior)
    ws_bytes = mod.workspace_size(T)
    ws_whole, ws_pay = _guarded(ws_bytes)
    ws_plain = mod.new_workspace(T)  # initialised by the library
    ws_pay.copy_(ws_plain.view(torch.uint8)[:ws_bytes])

    mod(dict(g, kv_cache=pool_g), out=out_g, gather_rows_out=rows_g, workspace=ws_pay)
    torch.cuda.synchronize()
    _say(f"[guards] {name} step done")

    assert _guards_intact(pool_whole, pool_bytes), "write outside kv_cache"
    assert _guards_intact(out_whole, T * sh.hidden * 2), "write outside out"
    assert _guards_intact(rows_whole, T * sh.n_prior * 4), "write outside gather_rows_out"
    assert _guards_intact(ws_whole, ws_bytes), "write outside the workspace"
    assert torch.equal(out_g, out_ref)
    assert torch.equal(rows_g, rows_ref)
    assert torch.equal(pool_g, pool_ref)
