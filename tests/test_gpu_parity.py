"""GPU parity of the HIP step against the fp64 oracle, through the C ABI.

Bars: gathered row addresses / mask bits and the set of written cache slots
bit-exact; the bf16 output and the bf16 written cache-row values within
|err| <= 2e-2 * RMS(reference) per element, plus half the bf16 spacing at the
reference value (the format's floor; it matters only beyond about 5 RMS),
with fp32 accumulation on the GPU.  Every token is compared.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from sparse_gather_mla_amd import Dims, MlaGatherDecode
from tests.harness import (TOL, bf16_half_ulp, bf16_to_f64, gpu_inputs, index_build_all, oracle_reference, rms,
                           token_slice, within_tol)
from workload import CONFIGS, MlaShape, Workload, make_inputs, pool_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _err_word(mod, ws=None):
    """The workspace's error word (MLA_GD_CHECK_* bits; right after the 256 zero bytes)."""
    ws = mod.workspace if ws is None else ws
    return int(ws.view(torch.int32)[256 // 4].item())


def _run_and_check(wl: Workload, tokens=None, fused=False, mutate=None, pool_check_rows=64, single=False):
    sh = wl.shape
    T, P, kvr = sh.n_tokens, sh.n_prior, sh.kv_row_dim
    _say(f"[parity] {wl.name} T={T} nh={sh.n_heads} P={P} fused={fused} single={single}")
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
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=T, fused=fused, single_launch=single)
    if single:
        assert mod.kernel_names(T) == ["k_step"]
    rows = torch.full((T, P), -7, dtype=torch.int32, device="cuda")
    out = mod(g, gather_rows_out=rows)
    torch.cuda.synchronize()
    _say(f"[parity] {wl.name} step done")
    assert _err_word(mod) == 0  # no wait of the fused or single-launch variant timed out

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
    excess = float(np.max(np.abs(got_out - ref["out"]) - bf16_half_ulp(ref["out"]))) / bound
    _say(f"[parity] {wl.name} out ({len(tokens)} of {T} tokens): max err {err:.3e} bound {bound:.3e} "
         f"err/bound {err / bound:.3f}, (err - bf16 floor)/bound {excess:.3f} (rms {rms(ref['out']):.3e})")
    assert ok
    # the worst token on its own scale too (a token whose output is much smaller
    # than the batch RMS must not hide behind the others)
    per_tok = [float(np.max(np.abs(got_out[i] - ref["out"][i]))) / (TOL * rms(ref["out"][i]))
               for i in range(len(tokens)) if rms(ref["out"][i]) > 0]
    if per_tok:
        worst = int(np.argmax(per_tok))
        _say(f"[parity] {wl.name} worst token {tokens[worst]}: err/(2e-2*rms of that token) {per_tok[worst]:.3f}")
    got_rows = bf16_to_f64(pool.view(-1, kvr)[slots[torch.as_tensor(tokens, device="cuda")]])
    ok, err, bound = within_tol(got_rows, ref["new_row"])
    _say(f"[parity] {wl.name} cache rows: max err {err:.3e} bound {bound:.3e} err/bound {err / bound:.3f}")
    assert ok
    # the GPU's stored row is a bf16 rounding of a value within tolerance of the exact row
    return out, ref, inp, g


@pytest.mark.parametrize("name", ["tiny", "ds32_slice", "batch32"])
def test_parity_small_and_medium(name):
    wl = next(w for w in CONFIGS if w.name == name)
    _run_and_check(wl)


# the 128-head configurations at full size, every token compared with the oracle
@pytest.mark.parametrize("name", ["fullhead64", "large128"])
def test_parity_full_head_all_tokens(name):
    wl = next(w for w in CONFIGS if w.name == name)
    _run_and_check(wl)


TINY_BASE = CONFIGS[0]

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


# The GEMV path's token passes: 2 tokens in a 2-token pass, 3 in a 4-token pass.
@pytest.mark.parametrize("T", [2, 3])
def test_parity_ragged_shape_gemv_token_passes(T):
    wl = replace(RAGGED, name=f"ragged_T{T}", shape=replace(RAGGED.shape, n_tokens=T), seed=177 + T)
    _run_and_check(wl)


# More than 128 tokens: two 128-token blocks on the matrix cores (the second
# one ragged) in every GEMM, the absorptions and the index build.
def test_parity_ragged_shape_two_token_blocks():
    wl = replace(RAGGED, name="ragged_T150", shape=replace(RAGGED.shape, n_tokens=150), seed=227)
    _run_and_check(wl)


# Steps of more than 3 tokens run the projections on the matrix cores.  Token
# counts that give one m-tile (4: the fewest, 12 padding rows; 9), a ragged
# block of two (21), a ragged block of four (37) and two blocks of four (70);
# the ragged shape also gives K not a multiple of the 32-wide k-step and
# column tiles with tails in every GEMM.
@pytest.mark.parametrize("T", [4, 9, 21, 37, 70])
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


# More than 64 heads: the core gives each wave one 16-head tile, 128 heads per
# workgroup.  72 heads leave half a tile and three waves without heads; 136
# heads make a second head block holding one half-empty tile.  Two tokens run
# the GEMV path, the others the matrix-core path.
@pytest.mark.parametrize("nh,T", [(72, 2), (72, 21), (136, 5)])
def test_parity_many_heads_one_tile_per_wave(nh, T):
    wl = replace(MANY_HEADS, name=f"ragged_heads{nh}_T{T}", shape=replace(MANY_HEADS.shape, n_tokens=T, n_heads=nh),
                 seed=300 + nh + T)
    _run_and_check(wl)


def _masked_splits(inp):
    gi = inp["gather_indices"]
    gi[1, :] = -1  # token 1: nothing valid, every split empty
    gi[2, 10:] = 2**30  # token 2: only its first ten entries valid, the later splits empty


# One token at dimensions other than the DeepSeek-V3.2 ones: the generic
# one-token kernels (the DeepSeek-V3.2 shape runs a copy compiled with its
# sizes as constants).
def test_parity_one_token_generic_kernels():
    wl = replace(RAGGED, name="ragged_T1", shape=replace(RAGGED.shape, n_tokens=1), seed=501)
    _run_and_check(wl)


# On the matrix-core path the core stores each split's output normalised by
# its own denominator; a split without a valid row must combine as zeros (and
# an all-masked token give a zero output row).  Both core shapes that do so:
# one 16-head tile (13 heads) and one tile per wave (72 heads).
@pytest.mark.parametrize("nh", [13, 72])
def test_matrix_core_empty_splits_and_all_masked_token(nh):
    base = MANY_HEADS if nh > 64 else RAGGED
    wl = replace(base, name=f"ragged_heads{nh}_T5_masked", shape=replace(base.shape, n_tokens=5, n_heads=nh),
                 seed=411 + nh)
    out, ref, inp, g = _run_and_check(wl, mutate=_masked_splits)
    assert torch.count_nonzero(out[1]).item() == 0


# 72-wide value heads give five 16-row output tiles: with few (head, token
# block) pairs the output absorption splits them over two workgroups per pair,
# the second holding one tile (three of its waves idle), and K5 = 1440 leaves
# A5 padding.
def test_parity_output_absorption_parts():
    wl = replace(RAGGED, name="ragged_dv72_T21", shape=replace(RAGGED.shape, n_tokens=21, v_head_dim=72), seed=121)
    _run_and_check(wl)


# ---------------------------------------------------------------------------
# the fused variant: kv rows, absorption and core in one launch (<= 16 heads, <= 3 tokens)
# ---------------------------------------------------------------------------
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
    assert _err_word(mod) == 0
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


# more than 64 heads: 64 core splits of 2560 rows, the most row ids the
# 128-head core stages; two tokens (GEMV path) and five (matrix cores)
MAX_PRIOR_WIDE = replace(MANY_HEADS, name="heads72_max_prior",
                         shape=replace(MANY_HEADS.shape, n_tokens=2, n_heads=72, n_prior=163840,
                                       max_blocks_per_seq=11250),
                         contexts=(170000, 179000), context_range=None, n_duplicates=1000, n_future=1000, seed=2103)


@pytest.mark.parametrize("T", [2, 5])
def test_parity_largest_n_prior_many_heads(T):
    wl = MAX_PRIOR_WIDE if T == 2 else replace(MAX_PRIOR_WIDE, name="heads72_max_prior_T5",
                                                shape=replace(MAX_PRIOR_WIDE.shape, n_tokens=5),
                                                contexts=(170000, 179000, 171000, 175000, 163900), seed=2104)
    _run_and_check(wl)


def test_parity_largest_token_count():
    _run_and_check(MAX_TOKENS)


# ---------------------------------------------------------------------------
# several tokens of one sequence in one step (multi-token / speculative
# decode): tokens of a sequence share its block-table row through token_seq,
# sit at its last positions, and each selects every other one of them
# (earlier ones read this step's rows, later ones are masked)
# ---------------------------------------------------------------------------
def _mt(base, name, T, k, seed, **shape_kw):
    return replace(base, name=name, shape=replace(base.shape, n_tokens=T, **shape_kw), contexts=None,
                   context_range=base.context_range or (60, 120), tokens_per_seq=k, seed=seed)


MT_GEMV = _mt(TINY_BASE, "tiny_mt_T3_k3", 3, 3, 3005)              # GEMV path: one sequence of 3
MULTI_TOKEN = [
    _mt(TINY_BASE, "tiny_mt_T6_k3", 6, 3, 3001),                      # matrix-core path, fewest tokens
    MT_GEMV,
    _mt(RAGGED, "ragged_mt_T21_k3", 21, 3, 3002),                     # matrix-core path
    _mt(MANY_HEADS, "heads40_mt_T20_k4", 20, 4, 3003),                # row-split core
    _mt(next(c for c in CONFIGS if c.name == "batch32"), "batch32_mt_k4", 32, 4, 3004),  # DeepSeek dims
]


@pytest.mark.parametrize("wl", MULTI_TOKEN, ids=[w.name for w in MULTI_TOKEN])
def test_parity_multi_token_sequences(wl):
    out, ref, inp, g = _run_and_check(wl)
    assert int(inp["token_seq"].max()) == wl.shape.n_tokens // wl.tokens_per_seq - 1


def test_parity_multi_token_fused_variant():
    _run_and_check(MT_GEMV, fused=True)


def test_multi_token_batch_matches_successive_single_token_steps():
    """The batched step equals the tokens run one by one in position order,
    each single-token step seeing the rows the earlier ones wrote."""
    wl = MULTI_TOKEN[0]
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    pool0 = g["kv_cache"].clone()
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    batched = mod(g).clone()
    pool_batched = g["kv_cache"].clone()
    g["kv_cache"].copy_(pool0)
    seq = inp["token_seq"].long()
    for t in torch.argsort(inp["positions"], stable=True).tolist():
        one = token_slice(g, [t])
        del one["token_seq"]
        one["block_table"] = g["block_table"][seq[t]:seq[t] + 1].contiguous()
        one["kv_cache"] = g["kv_cache"]
        o = mod(one)
        torch.cuda.synchronize()
        ok, err, bound = within_tol(bf16_to_f64(o[0]), bf16_to_f64(batched[t]))
        _say(f"[multi-token] token {t}: successive vs batched max err {err:.3e} bound {bound:.3e}")
        assert ok
    ok, err, bound = within_tol(bf16_to_f64(g["kv_cache"]), bf16_to_f64(pool_batched))
    assert ok


# ---------------------------------------------------------------------------
# A score far above the rest, late in a split: for three tokens one gathered
# row, past the first 32-row chunk of its split, is replaced by the token's
# own head-0 query (from the oracle's front-fold) with the other heads' query
# directions projected out, scaled so that head 0 scores it +100 (log2 units)
# and every other head about 0.  The core's online softmax must move head 0's
# reference by about 95 units in mid-split (rescaling what it accumulated).
# Only one head sees the outsized score: a large |q||k| in many heads would
# turn the bf16 query tile's rounding into score errors of a tenth of a unit
# and fail the bar for any bf16-query design, so the case tests the softmax
# and nothing else.  The oracle reads the same pool.
# ---------------------------------------------------------------------------
FAR_SCORE = Workload(
    name="heads40_far_score",
    shape=MlaShape(n_tokens=32, hidden=1160, q_lora_rank=600, kv_lora_rank=128, qk_nope_head_dim=24,
                   qk_rope_head_dim=16, v_head_dim=40, n_heads=40, block_size=16, max_blocks_per_seq=48,
                   n_prior=512, softmax_scale=0.2, norm_eps=1e-6),
    seed=4242, context_range=(600, 760), n_duplicates=7, n_future=5,
)


def test_parity_one_far_larger_score_late_in_a_split():
    wl = FAR_SCORE
    sh = wl.shape
    r = sh.kv_lora_rank
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    flat = g["kv_cache"].view(-1, sh.kv_row_dim)
    rows = index_build_all(inp, sh.block_size)
    o64 = oracle.to_f64_inputs({k: v for k, v in inp.items() if k != "kv_cache"}, block_size=sh.block_size)
    w = {k: o64[k] for k in ("input_norm_w", "wq_a", "q_norm_w", "wq_b", "wkv_a", "kv_norm_w", "q_absorb_w",
                             "out_absorb_w", "o_proj_w")}
    placed = []
    for t in (0, 5, 31):
        q_lat, q_pe, _, _ = oracle.front_fold(o64["hidden_states"][t], w, o64["cos"][t], o64["sin"][t], sh.n_heads,
                                              sh.qk_nope_head_dim, sh.qk_rope_head_dim, r, sh.norm_eps)
        qall = np.concatenate([q_lat, q_pe], axis=1)
        basis, _ = np.linalg.qr(qall[1:].T)  # the other heads' query directions
        d = qall[0] - basis @ (basis.T @ qall[0])
        # head 0's score (log2 units) = softmax_scale * log2(e) * (q0 . row) = 100
        row = d * (100.0 / (sh.softmax_scale * 1.4426950408889634 * float(qall[0] @ d)))
        own = int(inp["slot_mapping"][t])
        # a position in the second half of a 64-row split; its row is selected nowhere else
        j = next(j for j in range(96, sh.n_prior) if j % 64 >= 32 and rows[t, j] >= 0 and rows[t, j] != own
                 and int(np.count_nonzero(rows[t] == rows[t, j])) == 1)
        flat[int(rows[t, j])] = torch.from_numpy(row).to(torch.bfloat16).cuda()
        placed.append((t, j, int(rows[t, j])))
    pool_cpu = g["kv_cache"].cpu()
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens)
    out = mod(g)
    torch.cuda.synchronize()
    # the pool copy predates the step: the oracle overlays this step's rows itself
    ref = oracle_reference(wl, inp, list(range(sh.n_tokens)), pool_cpu=pool_cpu)
    ok, err, bound = within_tol(bf16_to_f64(out), ref["out"])
    _say(f"[far score] (token, position, row) {placed}: max err {err:.3e} bound {bound:.3e} err/bound {err / bound:.3f}")
    assert ok


# ---------------------------------------------------------------------------
# the single-launch variant: the whole step as one kernel (<= 3 tokens,
# <= 16 heads).  Its arithmetic is the fused variant's (the same phases,
# splits, reduction orders and four-wave core), so besides the oracle bar it
# must give the same bits; below a 512-wide latent also the separate kernels'.
# ---------------------------------------------------------------------------
_BATCH32 = next(c for c in CONFIGS if c.name == "batch32")
RAGGED13 = replace(RAGGED, name="ragged_nh13", shape=replace(RAGGED.shape, n_heads=13), seed=4401)
SINGLE_CASES = [
    TINY_BASE,
    next(c for c in CONFIGS if c.name == "ds32_slice"),
    replace(_BATCH32.with_tokens(3), name="batch32_T3"),
    replace(RAGGED13, name="ragged_nh13_T3", shape=replace(RAGGED13.shape, n_tokens=3), seed=4403),  # a 4-token pass
    replace(RAGGED13, name="ragged_nh13_T2", shape=replace(RAGGED13.shape, n_tokens=2), seed=4402),
    MT_GEMV,                                                                               # 1 sequence x 3 tokens
]


@pytest.mark.parametrize("wl", SINGLE_CASES, ids=[w.name for w in SINGLE_CASES])
def test_parity_single_launch(wl):
    out, ref, inp, g = _run_and_check(wl, single=True)
    # the fused variant on the same inputs (the step rewrites the same rows
    # with the same values) gives the same bits: the same phases, splits and
    # four-wave core.  (The separately launched core takes eight waves at a
    # 512-wide latent, so its score sums round in another order.)
    fz = MlaGatherDecode(Dims.from_shape(wl.shape), max_tokens=wl.shape.n_tokens, fused=True)
    assert fz.kernel_names(wl.shape.n_tokens)[2] == "k_absorb_core"
    out_fz = fz(g)
    torch.cuda.synchronize()
    assert torch.equal(out, out_fz)
    if wl.shape.kv_lora_rank < 512:  # the separate kernels' core has four waves too
        sep = MlaGatherDecode(Dims.from_shape(wl.shape), max_tokens=wl.shape.n_tokens)
        out_sep = sep(g)
        torch.cuda.synchronize()
        assert torch.equal(out, out_sep)


def test_single_launch_self_row_and_all_masked():
    """A token that selects its own position must see this step's row: the
    single launch's core waits for every kv-row workgroup before it reads a row id."""
    out, ref, inp, g = _run_and_check(TINY, single=True, mutate=_self_row_and_all_masked)
    assert torch.count_nonzero(out[1]).item() == 0


def test_single_launch_repeated_steps_of_varying_size():
    """One handle and workspace run steps of 8 (matrix-core path), 3, 1, 8, 1
    and 2 tokens in a row: flags of an earlier (larger) step never satisfy a
    later step's waits (the epoch advances every step, and the other path's
    steps leave the flag region alone), each step gives the bits of the fused
    variant (the separate kernels at 8 tokens), and no wait times out."""
    wl = _BATCH32.with_tokens(8)
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    single = MlaGatherDecode(Dims.from_shape(sh), max_tokens=8, single_launch=True)
    sep = MlaGatherDecode(Dims.from_shape(sh), max_tokens=8, fused=True)
    for T in (8, 3, 1, 8, 1, 2):
        sub = token_slice(g, list(range(T)))
        sub["kv_cache"] = g["kv_cache"]
        a = single(sub).clone()
        b = sep(sub).clone()
        torch.cuda.synchronize()
        _say(f"[single] steps of {T} tokens: equal {torch.equal(a, b)}")
        assert torch.equal(a, b)
    assert _err_word(single) == 0


def test_single_launch_noalloc_and_graph_replay():
    """The single launch through the allocation-free entry point (the static
    device array) and replayed from a captured graph, three times each: the
    same bits as the fused variant every time."""
    wl = CONFIGS[1]  # ds32_slice
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    g = gpu_inputs(wl, inp)
    dims = Dims.from_shape(sh)
    ref = MlaGatherDecode(dims, max_tokens=1, fused=True)(g).clone()
    single = MlaGatherDecode(dims, max_tokens=1, single_launch=True)
    graphed = MlaGatherDecode(dims, max_tokens=1, single_launch=True, graph=True)
    fixed = torch.empty_like(ref)
    for i in range(3):
        a = single(g, noalloc=True).clone()
        graphed(g, out=fixed)
        torch.cuda.synchronize()  # eager work and synchronisation between replays
        _say(f"[single] noalloc / graph replay {i}")
        assert torch.equal(a, ref) and torch.equal(fixed, ref)
    assert _err_word(graphed) == 0
