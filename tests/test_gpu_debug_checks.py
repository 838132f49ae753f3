"""Device-side checks of the caller's index data (MLA_GD_FLAG_DEBUG_CHECKS),
through the C ABI, on the GEMV path, the matrix-core path, the fused variant
and the single-launch variant.

Valid inputs give the same bits as a handle without the checks.  A block-table
column or block id out of range masks that entry (the index build and the
output then match the oracle on the inputs with the entry masked), an
out-of-range slot leaves the pool unwritten for that token, a shared slot is
reported; each sets its bit of the error word, and the next step returns
MLA_GD_E_DEVICE_CHECK without launching anything.
"""
import copy
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from sparse_gather_mla_amd import (MLA_GD_CHECK_BLOCK_RANGE, MLA_GD_CHECK_SLOT_RANGE, MLA_GD_CHECK_SLOT_SHARED,
                                   MLA_GD_CHECK_TABLE_COLUMN, Dims, MlaGatherDecode, MlaGdError)
from tests.harness import bf16_to_f64, gpu_inputs, index_build_all, oracle_reference, within_tol
from workload import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

TINY = CONFIGS[0]
TINY24 = replace(CONFIGS[0], name="tiny_T24", shape=replace(CONFIGS[0].shape, n_tokens=24),
                 contexts=None, context_range=(40, 120), seed=1024)
# path -> (workload, handle options)
PATHS = {"gemv": (TINY, {}), "mfma": (TINY24, {}), "fused": (TINY, {"fused": True}),
         "single": (TINY, {"single_launch": True})}
E_DEVICE_CHECK = 6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _handles(wl, opts):
    dims, T = Dims.from_shape(wl.shape), wl.shape.n_tokens
    return (MlaGatherDecode(dims, max_tokens=T, debug_checks=True, **opts),
            MlaGatherDecode(dims, max_tokens=T, **opts))


def _rows_buf(sh):
    return torch.full((sh.n_tokens, sh.n_prior), -7, dtype=torch.int32, device="cuda")


def _mask_entries(inp, t, pred):
    """Copy of inp with token t's causally valid entries g for which pred(g) holds set to -1."""
    ref = copy.deepcopy(inp)
    gi = ref["gather_indices"]
    pos = int(ref["positions"][t])
    n = 0
    for j in range(gi.shape[1]):
        g = int(gi[t, j])
        if 0 <= g <= pos and pred(g):
            gi[t, j] = -1
            n += 1
    return ref, n


def _check_masked_run(path, wl, opts, bad, ref, bit):
    """Run `bad` with the checks; it must index, and compute, as `ref` (the
    offending entries masked), report `bit`, and make the next step fail."""
    sh = wl.shape
    dbg, _ = _handles(wl, opts)
    g_bad = gpu_inputs(wl, bad)
    rows = _rows_buf(sh)
    out = dbg(g_bad, gather_rows_out=rows).clone()
    torch.cuda.synchronize()
    _say(f"[debug] {path} step done")
    assert np.array_equal(rows.cpu().numpy().astype(np.int64), index_build_all(ref, sh.block_size))
    assert torch.isfinite(out.float()).all()
    tokens = list(range(sh.n_tokens))
    oref = oracle_reference(wl, ref, tokens)
    ok, err, bound = within_tol(bf16_to_f64(out), oref["out"])
    _say(f"[debug] {path} out: max err {err:.3e} bound {bound:.3e}")
    assert ok
    # the next step reads the error word first and launches nothing
    with pytest.raises(MlaGdError) as ei:
        dbg(g_bad)
    assert ei.value.code == E_DEVICE_CHECK
    # the word is clear again: the same inputs report the same bit once more
    dbg(g_bad)
    assert dbg.debug_status() == bit
    assert dbg.debug_status() == 0


@pytest.mark.parametrize("path", list(PATHS))
def test_valid_inputs_same_bits_without_error(path):
    wl, opts = PATHS[path]
    sh = wl.shape
    _say(f"[debug] valid inputs, {path} T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    dbg, plain = _handles(wl, opts)
    pool0 = g["kv_cache"].clone()
    rows_d, rows_p = _rows_buf(sh), _rows_buf(sh)
    out_d = dbg(g, gather_rows_out=rows_d).clone()
    cache_d = g["kv_cache"].clone()
    g["kv_cache"].copy_(pool0)
    out_p = plain(g, gather_rows_out=rows_p)
    torch.cuda.synchronize()
    assert dbg.debug_status() == 0
    assert torch.equal(rows_d, rows_p)
    assert torch.equal(out_d, out_p)
    assert torch.equal(cache_d, g["kv_cache"])
    dbg(g)  # a second step passes the error-word read
    assert dbg.debug_status() == 0


@pytest.mark.parametrize("path", list(PATHS))
def test_block_id_out_of_range_is_masked_and_reported(path):
    wl, opts = PATHS[path]
    sh = wl.shape
    bs = sh.block_size
    _say(f"[debug] block id out of range, {path} T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    pos = int(inp["positions"][0])
    valid = [int(g) for g in inp["gather_indices"][0] if 0 <= int(g) <= pos]
    col = valid[0] // bs
    ref, n = _mask_entries(inp, 0, lambda g: g // bs == col)
    assert n > 0
    bad = copy.deepcopy(inp)
    bad["block_table"][0, col] = sh.n_blocks + 3
    # the last token: a negative block id in the logical block of its last valid entry
    t = sh.n_tokens - 1
    pos_t = int(inp["positions"][t])
    col_t = [int(g) for g in inp["gather_indices"][t] if 0 <= int(g) <= pos_t][-1] // bs
    ref, n_t = _mask_entries(ref, t, lambda g: g // bs == col_t)
    assert n_t > 0
    bad["block_table"][t, col_t] = -2
    _check_masked_run(path, wl, opts, bad, ref, MLA_GD_CHECK_BLOCK_RANGE)


@pytest.mark.parametrize("path", list(PATHS))
def test_block_table_column_out_of_range_is_masked_and_reported(path):
    """A position past the table (position // block_size >= max_blocks_per_seq)
    that passes the causal mask."""
    wl, opts = PATHS[path]
    sh = wl.shape
    span = sh.max_blocks_per_seq * sh.block_size
    _say(f"[debug] table column out of range, {path} T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    bad = copy.deepcopy(inp)
    gi = bad["gather_indices"]
    pos = int(bad["positions"][0])
    # entries that the later position would unmask stay masked
    gi[0][(gi[0] > pos)] = -1
    bad["positions"][0] = span + 5
    gi[0, 3] = span + 2
    gi[0, 7] = span + 5  # the token's own position
    ref, n = _mask_entries(bad, 0, lambda g: g >= span)
    assert n == 2
    _check_masked_run(path, wl, opts, bad, ref, MLA_GD_CHECK_TABLE_COLUMN)


@pytest.mark.parametrize("path", list(PATHS))
def test_slot_out_of_range_leaves_the_pool_unwritten(path):
    wl, opts = PATHS[path]
    sh = wl.shape
    kvr, T = sh.kv_row_dim, sh.n_tokens
    bad_t = T - 1
    _say(f"[debug] slot out of range, {path} T={T}")
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    dbg, plain = _handles(wl, opts)
    pool0 = g["kv_cache"].clone()
    g_bad = dict(g)
    g_bad["slot_mapping"] = g["slot_mapping"].clone()
    g_bad["slot_mapping"][bad_t] = sh.n_blocks * sh.block_size + 7
    rows = _rows_buf(sh)
    out_bad = dbg(g_bad, gather_rows_out=rows).clone()
    cache_bad = g["kv_cache"].clone()
    torch.cuda.synchronize()
    _say(f"[debug] {path} step done")
    assert dbg.debug_status() == MLA_GD_CHECK_SLOT_RANGE
    g["kv_cache"].copy_(pool0)
    out_ref = plain(g)
    torch.cuda.synchronize()
    # every other token's row is written as without the bad slot, nothing else
    slot = int(g["slot_mapping"][bad_t])
    expect = g["kv_cache"].clone()
    expect.view(-1, kvr)[slot] = pool0.view(-1, kvr)[slot]
    assert torch.equal(cache_bad, expect)
    # tokens that do not gather the unwritten row are unaffected
    assert torch.isfinite(out_bad.float()).all()
    r = rows.cpu().numpy()
    same = [u for u in range(T) if slot not in r[u]]
    assert len(same) >= T - 1
    idx = torch.as_tensor(same, device="cuda")
    assert torch.equal(out_bad[idx], out_ref[idx])


@pytest.mark.parametrize("path", list(PATHS))
def test_shared_slot_is_reported(path):
    wl, opts = PATHS[path]
    sh = wl.shape
    kvr = sh.kv_row_dim
    _say(f"[debug] shared slot, {path} T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    dbg, plain = _handles(wl, opts)
    pool0 = g["kv_cache"].clone()
    s0, s1 = int(g["slot_mapping"][0]), int(g["slot_mapping"][1])
    g_sh = dict(g)
    g_sh["slot_mapping"] = g["slot_mapping"].clone()
    g_sh["slot_mapping"][1] = s0
    dbg(g_sh)
    cache_sh = g["kv_cache"].clone()
    torch.cuda.synchronize()
    _say(f"[debug] {path} step done")
    assert dbg.debug_status() == MLA_GD_CHECK_SLOT_SHARED
    g["kv_cache"].copy_(pool0)
    plain(g)
    torch.cuda.synchronize()
    flat, ref = cache_sh.view(-1, kvr), g["kv_cache"].view(-1, kvr)
    # each element of the shared row is token 0's or token 1's; token 1's own slot is untouched
    assert bool(((flat[s0] == ref[s0]) | (flat[s0] == ref[s1])).all())
    assert torch.equal(flat[s1], pool0.view(-1, kvr)[s1])


def test_debug_checks_with_graph_replay():
    """With the graph flag the error word is read before each replay; index data
    changed in place (same pointers) reach the replayed kernels."""
    wl = TINY
    sh = wl.shape
    bs = sh.block_size
    _say(f"[debug] graph replay, T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    dims = Dims.from_shape(sh)
    mod = MlaGatherDecode(dims, max_tokens=sh.n_tokens, graph=True, debug_checks=True)
    plain = MlaGatherDecode(dims, max_tokens=sh.n_tokens)
    pool0 = g["kv_cache"].clone()
    out1 = mod(g).clone()
    out2 = mod(g).clone()
    torch.cuda.synchronize()
    assert mod.debug_status() == 0
    g["kv_cache"].copy_(pool0)
    ref = plain(g).clone()
    torch.cuda.synchronize()
    assert torch.equal(out1, ref) and torch.equal(out2, ref)
    # an out-of-range block id written in place into the captured block table
    pos = int(inp["positions"][0])
    col = [int(x) for x in inp["gather_indices"][0] if 0 <= int(x) <= pos][0] // bs
    masked, n = _mask_entries(inp, 0, lambda x: x // bs == col)
    assert n > 0
    g["block_table"][0, col] = sh.n_blocks + 3
    out3 = mod(g).clone()
    torch.cuda.synchronize()
    _say("[debug] graph replay with a bad block id done")
    assert mod.debug_status() == MLA_GD_CHECK_BLOCK_RANGE
    ok, err, bound = within_tol(bf16_to_f64(out3), oracle_reference(wl, masked, list(range(sh.n_tokens)))["out"])
    assert ok, (err, bound)
    mod(g)
    with pytest.raises(MlaGdError) as ei:
        mod(g)
    assert ei.value.code == E_DEVICE_CHECK


def test_sequence_id_out_of_range_is_masked_and_reported():
    """Several tokens per sequence (token_seq): a token whose sequence id lies
    outside [0, n_tokens) has every entry masked (the block table is never
    read for it) and MLA_GD_CHECK_SEQ_RANGE is reported."""
    from sparse_gather_mla_amd import MLA_GD_CHECK_SEQ_RANGE

    wl = replace(CONFIGS[0], name="tiny_mt_dbg", shape=replace(CONFIGS[0].shape, n_tokens=6), contexts=None,
                 context_range=(60, 120), tokens_per_seq=3, seed=3101)
    sh = wl.shape
    _say(f"[debug] sequence id out of range, T={sh.n_tokens}")
    inp = make_inputs(wl, with_pool=False)
    bad = copy.deepcopy(inp)
    bad["token_seq"][1] = sh.n_tokens  # past the last allowed row
    ref, n = _mask_entries(inp, 1, lambda g: True)
    assert n > 0
    _check_masked_run("gemv", wl, {}, bad, ref, MLA_GD_CHECK_SEQ_RANGE)
