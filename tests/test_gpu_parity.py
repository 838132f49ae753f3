"""GPU parity of the HIP step against the fp64 oracle, through the C ABI.

Bars: gathered row addresses / mask bits and the set of written cache slots
bit-exact; the bf16 output and the bf16 written cache-row values within
max |err| <= 2e-2 * RMS(reference) (fp32 accumulation on the GPU).
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from sparse_gather_mla_amd import Dims, MlaGatherDecode
from tests.harness import (TOL, bf16_to_f64, gpu_inputs, index_build_all, oracle_reference, rms,
                           token_slice, within_tol)
from workload import CONFIGS, MlaShape, Workload, make_inputs, pool_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_and_check(wl: Workload, tokens=None, fused=False, mutate=None, pool_check_rows=64):
    sh = wl.shape
    T, P, kvr = sh.n_tokens, sh.n_prior, sh.kv_row_dim
    _say(f"[parity] {wl.name} T={T} nh={sh.n_heads} P={P} fused={fused}")
    inp = make_inputs(wl, with_pool=False)
    if mutate is not None:
        mutate(inp)
    g = gpu_inputs(wl, inp)
    pool = g["kv_cache"]
    flat = pool.view(-1, kvr)
    # the GPU-filled pool is the generator's pool
    probe = np.random.default_rng(0).integers(0, flat.shape[0], size=pool_check_rows)
    assert torch.equal(flat[torch.from_numpy(probe).cuda()].cpu(), pool_rows(wl, probe))
    before = pool.clone()
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=T, fused=fused)
    rows = torch.full((T, P), -7, dtype=torch.int32, device="cuda")
    out = mod(g, gather_rows_out=rows)
    torch.cuda.synchronize()
    _say(f"[parity] {wl.name} step done")

    # index build: bit-exact for every token
    ref_rows = index_build_all(inp, sh.block_size)
    assert np.array_equal(rows.cpu().numpy().astype(np.int64), ref_rows)

    # cache: only the slot rows changed
    slots = g["slot_mapping"].long()
    after = pool.clone()
    after.view(-1, kvr)[slots] = before.view(-1, kvr)[slots]
    assert torch.equal(after, before), "cache rows other than slot_mapping were modified"
    del after

    # values on the checked tokens
    tokens = list(range(T)) if tokens is None else list(tokens)
    ref = oracle_reference(wl, inp, tokens)
    got_out = bf16_to_f64(out[torch.as_tensor(tokens, device="cuda")])
    ok, err, bound = within_tol(got_out, ref["out"])
    _say(f"[parity] {wl.name} out: max err {err:.3e} bound {bound:.3e} (rms {rms(ref['out']):.3e})")
    assert ok
    got_rows = bf16_to_f64(pool.view(-1, kvr)[slots[torch.as_tensor(tokens, device="cuda")]])
    ok, err, bound = within_tol(got_rows, ref["new_row"])
    _say(f"[parity] {wl.name} cache rows: max err {err:.3e} bound {bound:.3e}")
    assert ok
    # the GPU's stored row is a bf16 rounding of a value within tolerance of the exact row
    return out, ref, inp, g


@pytest.mark.parametrize("name", ["tiny", "ds32_slice", "batch32"])
def test_parity_small_and_medium(name):
    wl = next(w for w in CONFIGS if w.name == name)
    _run_and_check(wl)


@pytest.mark.parametrize("name,tokens", [("fullhead64", [0, 17, 40, 63]), ("large128", [0, 77, 127])])
def test_parity_full_head_sampled_tokens(name, tokens):
    wl = next(w for w in CONFIGS if w.name == name)
    _run_and_check(wl, tokens=tokens)


# ---------------------------------------------------------------------------
# a ragged shape: several column tiles with tails, 2 head groups (16 + 4),
# n_prior not a multiple of the row chunk
# ---------------------------------------------------------------------------
RAGGED = Workload(
    name="ragged",
    shape=MlaShape(n_tokens=5, hidden=1160, q_lora_rank=600, kv_lora_rank=64, qk_nope_head_dim=24,
                   qk_rope_head_dim=16, v_head_dim=40, n_heads=20, block_size=16, max_blocks_per_seq=12,
                   n_prior=100, softmax_scale=0.2, norm_eps=1e-6),
    seed=77, context_range=(101, 180), n_duplicates=7, n_future=5,
)


def test_parity_ragged_shape():
    _run_and_check(RAGGED)


# The GEMV path's token passes: 3 tokens in a 4-token pass, 8 in a full one.
@pytest.mark.parametrize("T", [3, 8])
def test_parity_ragged_shape_gemv_token_passes(T):
    wl = replace(RAGGED, name=f"ragged_T{T}", shape=replace(RAGGED.shape, n_tokens=T), seed=177 + T)
    _run_and_check(wl)


# More than 128 tokens: two 128-token blocks on the matrix cores (the second
# one ragged) in every GEMM, the absorptions and the index build.
def test_parity_ragged_shape_two_token_blocks():
    wl = replace(RAGGED, name="ragged_T150", shape=replace(RAGGED.shape, n_tokens=150), seed=227)
    _run_and_check(wl, tokens=[0, 63, 127, 128, 149])


# Steps of more than 8 tokens run the projections on the matrix cores.  Token
# counts that give one m-tile (9), a ragged block of two (21), a ragged block
# of four (37) and two blocks of four (70); the ragged shape also gives K not
# a multiple of the 32-wide k-step and column tiles with tails in every GEMM.
@pytest.mark.parametrize("T", [9, 21, 37, 70])
def test_parity_ragged_shape_matrix_core_path(T):
    wl = replace(RAGGED, name=f"ragged_T{T}", shape=replace(RAGGED.shape, n_tokens=T), seed=77 + T)
    _run_and_check(wl)


# More than 16 heads with a latent width of 128 or more run the row-split
# core: 40 heads leave the third head tile half full and the fourth empty;
# kv_row = 144 does not fill the last 32-wide k-step.  Both projection paths.
MANY_HEADS = Workload(
    name="ragged_heads40",
    shape=MlaShape(n_tokens=5, hidden=1160, q_lora_rank=600, kv_lora_rank=128, qk_nope_head_dim=24,
                   qk_rope_head_dim=16, v_head_dim=40, n_heads=40, block_size=16, max_blocks_per_seq=12,
                   n_prior=100, softmax_scale=0.2, norm_eps=1e-6),
    seed=91, context_range=(101, 180), n_duplicates=7, n_future=5,
)


@pytest.mark.parametrize("T", [5, 21])
def test_parity_many_heads_row_split_core(T):
    wl = replace(MANY_HEADS, name=f"ragged_heads40_T{T}", shape=replace(MANY_HEADS.shape, n_tokens=T), seed=91 + T)
    _run_and_check(wl)


# 72-wide value heads give five 16-row output tiles: with few (head, token
# block) pairs the output absorption splits them over two workgroups per pair,
# the second holding one tile (three of its waves idle), and K5 = 1440 leaves
# A5 padding.
def test_parity_output_absorption_parts():
    wl = replace(RAGGED, name="ragged_dv72_T21", shape=replace(RAGGED.shape, n_tokens=21, v_head_dim=72), seed=121)
    _run_and_check(wl)


# ---------------------------------------------------------------------------
# the fused variant: kv rows, absorption and core in one launch (<= 16 heads, <= 8 tokens)
# ---------------------------------------------------------------------------
def _fused_error_word(mod):
    # the fused counters sit right after the workspace's first 256 bytes, 64 bytes apart;
    # the second one is the error flag a timed-out wait raises
    return int(mod.workspace.view(torch.int32)[(256 + 64) // 4].item())


@pytest.mark.parametrize("name", ["tiny", "ds32_slice"])
def test_parity_fused_variant(name):
    wl = next(w for w in CONFIGS if w.name == name)
    sh = wl.shape
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens, fused=True)
    assert "k_absorb_core" in mod.kernel_names(sh.n_tokens)
    _run_and_check(wl, fused=True)


def test_fused_variant_self_row_and_all_masked():
    """A token that selects its own position must see this step's row: the
    fused core waits for the kv-row counter before it reads the cache."""
    out, ref, inp, g = _run_and_check(TINY, fused=True, mutate=_self_row_and_all_masked)
    assert torch.count_nonzero(out[1]).item() == 0


def test_fused_variant_counters_and_repeat():
    """Repeated fused steps give the same bits and never raise the wait-timeout flag."""
    wl = TINY
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens, fused=True)
    sep = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    outs = [mod(g).clone() for _ in range(3)]
    ref = sep(g).clone()
    torch.cuda.synchronize()
    assert _fused_error_word(mod) == 0
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    ok, err, bound = within_tol(bf16_to_f64(outs[0]), bf16_to_f64(ref))
    assert ok, (err, bound)


def test_parity_tiny_shape_matrix_core_path():
    """Smallest dims (hidden 256, kv_lora_rank 64, 4 heads) with 24 tokens and the tiny recipe."""
    wl = replace(CONFIGS[0], name="tiny_T24", shape=replace(CONFIGS[0].shape, n_tokens=24),
                 contexts=None, context_range=(40, 120), seed=1024)
    _run_and_check(wl)


def _mostly_future(inp):
    gi = inp["gather_indices"]
    pos = int(inp["positions"][0])
    n = gi.shape[1]
    gi[0, 200:] = pos + 1 + torch.arange(n - 200, dtype=gi.dtype) % 50  # masked (future)


def test_one_token_mostly_masked_many_splits():
    """ds32_slice shape (one token: 64 row splits of 32) with only the first 200
    entries valid, so most splits hold no valid row and combine as zeros."""
    wl = next(c for c in CONFIGS if c.name == "ds32_slice")
    _run_and_check(wl, mutate=_mostly_future)


# ---------------------------------------------------------------------------
# special inputs on the tiny shape
# ---------------------------------------------------------------------------
TINY = CONFIGS[0]


def _self_row_and_all_masked(inp):
    gi = inp["gather_indices"]
    gi[0, 4] = inp["positions"][0]  # token 0 selects its own position (this step's row)
    gi[1, :] = -1  # token 1: nothing valid
    gi[1, 3] = 2**30


def test_self_row_selected_and_all_masked_token():
    out, ref, inp, g = _run_and_check(TINY, mutate=_self_row_and_all_masked)
    assert torch.count_nonzero(out[1]).item() == 0


def _all_duplicates(inp):
    inp["gather_indices"][:, :] = inp["gather_indices"][:, :1].clone().clamp(max=inp["positions"].min())


def test_all_entries_duplicate():
    _run_and_check(TINY, mutate=_all_duplicates)


def _far_future(inp):
    gi = inp["gather_indices"]
    gi[0, 0] = 2**30
    gi[1, 1] = 2**31 - 1
    gi[1, 2] = -5


def test_future_indices_past_the_table():
    _run_and_check(TINY, mutate=_far_future)


def test_nan_poisoned_masked_rows_do_not_leak():
    """Rows that masked (future) entries would resolve to hold NaN; the output is unaffected."""
    wl = TINY
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    pool = g["kv_cache"].view(-1, sh.kv_row_dim)
    bt = inp["block_table"].numpy()
    for t in range(sh.n_tokens):
        pos = int(inp["positions"][t])
        fut = [int(bt[t, q // sh.block_size]) * sh.block_size + q % sh.block_size
               for q in range(pos + 1, sh.max_blocks_per_seq * sh.block_size)]
        pool[torch.tensor(fut, device="cuda")] = float("nan")
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    out = mod(g)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ref = oracle_reference(wl, inp, list(range(sh.n_tokens)))
    ok, err, bound = within_tol(bf16_to_f64(out), ref["out"])
    assert ok, (err, bound)


def test_fewer_tokens_than_max_and_repeat_is_idempotent():
    """A handle sized for 4 tokens runs steps of 2 and 1 tokens; repeating a step
    gives the same bits (it rewrites the same slots with the same values)."""
    wl = TINY
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=4)
    out1 = mod(g).clone()
    cache1 = g["kv_cache"].clone()
    out2 = mod(g).clone()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(cache1, g["kv_cache"])
    one = token_slice(g, [1])
    one["kv_cache"] = g["kv_cache"]
    out3 = mod(one)
    torch.cuda.synchronize()
    ref = oracle_reference(wl, inp, [0, 1])
    ok, err, bound = within_tol(bf16_to_f64(out3), ref["out"][1:2])
    assert ok, (err, bound)


def test_graph_replay_matches_direct_launches_and_recaptures():
    """With the graph flag the step is captured once and replayed; it gives the
    same bits as direct launches, replays repeatedly, and captures again when
    an output pointer changes (the new buffer receives the result)."""
    wl = CONFIGS[1]  # ds32_slice
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    direct = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    graphed = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens, graph=True)
    ref = direct(g).clone()
    fixed = torch.empty_like(ref)
    outs = []
    for _ in range(3):
        graphed(g, out=fixed)  # same arguments: the captured graph is replayed
        outs.append(fixed.clone())
        torch.cuda.synchronize()  # eager work and synchronisation between replays
    other = torch.zeros_like(ref)
    graphed(g, out=other)
    torch.cuda.synchronize()
    for o in outs + [other]:
        assert torch.equal(o, ref)


# ---------------------------------------------------------------------------
# the documented size limits, on the small dims: n_prior = 262144 (64 core
# splits of 4096 rows, the most row ids a core workgroup stages) and
# max_tokens = 4096 (32 blocks of 128 tokens on the matrix cores)
# ---------------------------------------------------------------------------
MAX_PRIOR = replace(CONFIGS[0], name="tiny_max_prior",
                    shape=replace(CONFIGS[0].shape, n_tokens=1, n_prior=262144, max_blocks_per_seq=18760),
                    contexts=(300000,), context_range=None, n_duplicates=1000, n_future=1000, seed=2101)
MAX_TOKENS = replace(CONFIGS[0], name="tiny_max_tokens", shape=replace(CONFIGS[0].shape, n_tokens=4096),
                     contexts=None, context_range=(40, 120), seed=2102)


def test_parity_largest_n_prior():
    _run_and_check(MAX_PRIOR)


def test_parity_largest_token_count():
    _run_and_check(MAX_TOKENS, tokens=[0, 1, 2047, 4095])
