"""Pins of the fp64 oracle against things other than itself.

Each test ties a part of the oracle to a closed form, an independent library
routine, a hand-worked fixture, or an invariant of the mathematics, chosen so
that a plausible slip (a dropped term, a transposed operand, a wrong sign or
index, dedup of duplicates, reading masked rows) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workload import CONFIGS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_case(seed=0, T=2, H=48, Q=24, r=16, dn=8, dr=8, dv=12, nh=3, bs=4, MB=6, P=10,
               scale=None, positions=None):
    """A random small step with every tensor drawn here (not from the generator)."""
    rng = np.random.default_rng(seed)
    n_blocks = T * MB
    inp = dict(
        hidden_states=rng.standard_normal((T, H)),
        input_norm_w=1 + 0.1 * rng.standard_normal(H),
        wq_a=rng.standard_normal((H, Q)) / math.sqrt(H),
        q_norm_w=1 + 0.1 * rng.standard_normal(Q),
        wq_b=rng.standard_normal((Q, nh * (dn + dr))) / math.sqrt(Q),
        wkv_a=rng.standard_normal((H, r + dr)) / math.sqrt(H),
        kv_norm_w=1 + 0.1 * rng.standard_normal(r),
        q_absorb_w=rng.standard_normal((nh, dn, r)) / math.sqrt(r),
        out_absorb_w=rng.standard_normal((nh, dv, r)) / math.sqrt(r),
        o_proj_w=rng.standard_normal((nh * dv, H)) / math.sqrt(nh * dv),
        n_heads=nh, qk_nope_head_dim=dn, qk_rope_head_dim=dr, kv_lora_rank=r,
        softmax_scale=(1 / math.sqrt(dn + dr)) if scale is None else scale,
        norm_eps=1e-6, kv_cache_block_size=bs,
    )
    if positions is None:
        positions = rng.integers(P, MB * bs - 1, size=T)
    positions = np.asarray(positions, dtype=np.int64)
    ang = positions[:, None] * np.power(10000.0, -2.0 * np.arange(dr // 2) / dr)[None, :]
    inp["cos"], inp["sin"] = np.cos(ang), np.sin(ang)
    bt = rng.permutation(n_blocks).reshape(T, MB)
    inp["block_table"] = bt
    inp["positions"] = positions
    inp["slot_mapping"] = bt[np.arange(T), positions // bs] * bs + positions % bs
    gi = np.stack([rng.choice(int(p) + 1, size=P, replace=False) for p in positions])
    inp["gather_indices"] = gi
    pool = rng.standard_normal((n_blocks * bs, r + dr))
    return inp, pool


def _run(inp, pool, trace=None):
    return oracle.mla_gather_decode_step(inp, oracle.dense_row_reader(pool), trace=trace)


# ---------------------------------------------------------------------------
# elementary pieces
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_conversion():
    """bf16 rounding equals torch's float32 -> bfloat16 cast (round to nearest even)."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    # exact ties: low 16 bits = 0x8000, with odd and even kept parts
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32) + np.float32(0)
    ties = np.concatenate([ties, (np.array([0x3F808000, 0x3F818000, 0xBF808000], np.uint32)).view(np.float32)])
    for arr in (f32, ties):
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        got = oracle.bf16_round(arr.astype(np.float64))
        assert np.array_equal(got, ref)


def test_rms_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 300)) * 3
    g = 1 + 0.1 * rng.standard_normal(300)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (300,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), ref, rtol=1e-14, atol=0)
    # scale invariance with eps = 0, and the eps term inside the root
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, g, 0.0), oracle.rms_norm(x, g, 0.0), rtol=1e-13)
    one = np.zeros(4)
    one[2] = 1.0
    np.testing.assert_allclose(oracle.rms_norm(one, np.ones(4), 0.75), one / math.sqrt(0.25 + 0.75))


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 16))
    theta = rng.uniform(-10, 10, size=8)
    c, s = np.cos(theta), np.sin(theta)
    np.testing.assert_array_equal(oracle.rope_interleaved(x, np.ones(8), np.zeros(8)), x)
    y = oracle.rope_interleaved(x, c, s)
    np.testing.assert_allclose(y[:, 0::2] ** 2 + y[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2, rtol=1e-13)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * theta)  # adjacent pair as one complex number
    np.testing.assert_allclose(y[:, 0::2], z.real, atol=1e-13)
    np.testing.assert_allclose(y[:, 1::2], z.imag, atol=1e-13)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    dr = 16
    q, k = rng.standard_normal(dr), rng.standard_normal(dr)
    freq = np.power(10000.0, -2.0 * np.arange(dr // 2) / dr)

    def rot(v, p):
        return oracle.rope_interleaved(v, np.cos(p * freq), np.sin(p * freq))

    a = rot(q, 1000) @ rot(k, 990)
    b = rot(q, 37) @ rot(k, 27)
    assert abs(a - b) < 1e-10
    assert abs(rot(q, 37) @ rot(k, 26) - b) > 1e-6


def test_index_build_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "index_build_small.json")) as f:
        g = json.load(f)
    bt = np.asarray(g["block_table"])
    for t, pos in enumerate(g["positions"]):
        got = [oracle.resolve_row(x, pos, bt[t], g["block_size"]) for x in g["gather_indices"][t]]
        assert got == g["rows"][t]


def _case_with_tables(block_table, token_seq, positions, gather_indices, block_size, seed=0, n_blocks=None,
                      H=40, Q=16, r=16, dn=8, dr=8, dv=12, nh=3):
    """Random weights and pool around given index tensors (several tokens may
    share a sequence's block-table row through token_seq)."""
    rng = np.random.default_rng(seed)
    bt = np.asarray(block_table, dtype=np.int64)
    seq = np.asarray(token_seq, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    T = len(pos)
    if n_blocks is None:
        n_blocks = int(bt.max()) + 1
    inp = dict(
        hidden_states=rng.standard_normal((T, H)),
        input_norm_w=1 + 0.1 * rng.standard_normal(H),
        wq_a=rng.standard_normal((H, Q)) / math.sqrt(H),
        q_norm_w=1 + 0.1 * rng.standard_normal(Q),
        wq_b=rng.standard_normal((Q, nh * (dn + dr))) / math.sqrt(Q),
        wkv_a=rng.standard_normal((H, r + dr)) / math.sqrt(H),
        kv_norm_w=1 + 0.1 * rng.standard_normal(r),
        q_absorb_w=rng.standard_normal((nh, dn, r)) / math.sqrt(r),
        out_absorb_w=rng.standard_normal((nh, dv, r)) / math.sqrt(r),
        o_proj_w=rng.standard_normal((nh * dv, H)) / math.sqrt(nh * dv),
        n_heads=nh, qk_nope_head_dim=dn, qk_rope_head_dim=dr, kv_lora_rank=r,
        softmax_scale=1 / math.sqrt(dn + dr), norm_eps=1e-6, kv_cache_block_size=block_size,
    )
    ang = pos[:, None] * np.power(10000.0, -2.0 * np.arange(dr // 2) / dr)[None, :]
    inp["cos"], inp["sin"] = np.cos(ang), np.sin(ang)
    inp["block_table"] = bt
    inp["token_seq"] = seq
    inp["positions"] = pos
    inp["slot_mapping"] = bt[seq, pos // block_size] * block_size + pos % block_size
    inp["gather_indices"] = np.asarray(gather_indices, dtype=np.int64)
    pool = rng.standard_normal((n_blocks * block_size, r + dr))
    return inp, pool


def test_index_build_multi_token_fixture():
    """Several tokens of one sequence: each resolves through its sequence's
    table row; earlier tokens' positions are valid, later ones masked."""
    with open(os.path.join(GOLDEN, "index_build_multi_token.json")) as f:
        g = json.load(f)
    inp, pool = _case_with_tables(g["block_table"], g["token_seq"], g["positions"], g["gather_indices"],
                                  g["block_size"])
    assert inp["slot_mapping"].tolist() == g["slot_mapping"]
    res = _run(inp, pool)
    assert res["rows"].tolist() == g["rows"]


def test_multi_token_batch_equals_successive_single_token_steps():
    """Two sequences, three and two tokens at consecutive positions, each
    selecting its sequence's other tokens' positions (and masked later ones):
    one batched step equals single-token steps run in position order, each
    writing its row into the pool before the next one runs."""
    bs, MB = 4, 6
    rng = np.random.default_rng(8)
    bt = rng.permutation(2 * MB).reshape(2, MB)
    seq = np.array([0, 1, 0, 1, 0])
    pos = np.array([13, 9, 14, 10, 15])
    P = 9
    gi = np.empty((5, P), dtype=np.int64)
    for t in range(5):
        mine = [int(p) for p, s in zip(pos, seq) if s == seq[t]]  # its sequence's tokens, earlier and later
        rest = rng.choice(int(pos[t]) - 2, size=P - len(mine), replace=False)
        row = np.concatenate([mine, rest])
        rng.shuffle(row)
        gi[t] = row
    inp, pool = _case_with_tables(bt, seq, pos, gi, bs, seed=3, n_blocks=2 * MB)
    batched = _run(inp, pool)
    cur = pool.copy()
    per_token = ("hidden_states", "cos", "sin", "slot_mapping", "positions", "gather_indices")
    for t in np.argsort(pos, kind="stable"):
        one = {k: (v[[t]] if k in per_token else v) for k, v in inp.items() if k not in ("token_seq", "block_table")}
        one["block_table"] = bt[[seq[t]]]
        res = _run(one, cur)
        assert np.array_equal(res["rows"][0], batched["rows"][t])
        np.testing.assert_allclose(res["out"][0], batched["out"][t], rtol=1e-12, atol=1e-14)
        assert np.array_equal(res["stored_row"][0], batched["stored_row"][t])
        cur[int(inp["slot_mapping"][t])] = res["stored_row"][0]
    # the case exercises the cross-token reads: without the pool updates
    # between the single-token steps, the later tokens' outputs change
    changed = 0
    for t in range(5):
        one = {k: (v[[t]] if k in per_token else v) for k, v in inp.items() if k not in ("token_seq", "block_table")}
        one["block_table"] = bt[[seq[t]]]
        stale = _run(one, pool)
        changed += not np.allclose(stale["out"][0], batched["out"][t], rtol=1e-9)
    assert changed == 3  # every token but the first of each sequence


# ---------------------------------------------------------------------------
# layouts of the projections (one-hot probes with closed forms)
# ---------------------------------------------------------------------------

def test_weight_orientation_and_row_layout_one_hot():
    """x = one-hot e_i with unit gammas and eps = 0 gives x_hat = sqrt(H) e_i, so the
    kv row is sqrt(H) * wkv_a[i, :]: latent part normalised, rotary part verbatim."""
    inp, _ = _tiny_case(seed=5)
    H, r, dr = 48, 16, 8
    w = {k: inp[k] for k in ("wq_a", "wq_b", "wkv_a", "q_absorb_w")}
    w.update(input_norm_w=np.ones(H), q_norm_w=np.ones(24), kv_norm_w=np.ones(r))
    i = 11
    x = np.zeros(H)
    x[i] = 3.0
    _, _, _, row = oracle.front_fold(x, w, np.ones(dr // 2), np.zeros(dr // 2), 3, 8, dr, r, 0.0)
    kv = math.sqrt(H) * inp["wkv_a"][i]
    np.testing.assert_allclose(row[r:], kv[r:], rtol=1e-13)
    np.testing.assert_allclose(row[:r], kv[:r] / np.sqrt(np.mean(kv[:r] ** 2)), rtol=1e-13)


def test_wq_b_columns_are_head_major_nope_then_rope():
    """wq_b with column c equal to (c + 1) * u: q[h, k] = (c_q . u) * (h*(dn+dr) + k + 1),
    nope entries first within a head."""
    inp, _ = _tiny_case(seed=6)
    nh, dn, dr, r, Q, H = 3, 8, 8, 16, 24, 48
    rng = np.random.default_rng(7)
    u = rng.standard_normal(Q)
    wq_b = u[:, None] * (np.arange(nh * (dn + dr)) + 1.0)[None, :]
    w = dict(input_norm_w=np.ones(H), wq_a=inp["wq_a"], q_norm_w=np.ones(Q), wq_b=wq_b,
             wkv_a=inp["wkv_a"], kv_norm_w=np.ones(r), q_absorb_w=inp["q_absorb_w"])
    x = rng.standard_normal(H)
    _, q_pe, q_nope, _ = oracle.front_fold(x, w, np.ones(dr // 2), np.zeros(dr // 2), nh, dn, dr, r, 0.0)
    q_a = oracle.rms_norm(x, np.ones(H), 0.0) @ inp["wq_a"]
    a = oracle.rms_norm(q_a, np.ones(Q), 0.0) @ u
    for h in range(nh):
        base = h * (dn + dr) + 1
        np.testing.assert_allclose(q_nope[h], a * (base + np.arange(dn)), rtol=1e-12)
        np.testing.assert_allclose(q_pe[h], a * (base + dn + np.arange(dr)), rtol=1e-12)


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------

def _explicit_mha_out(inp, res, trace, t, pool):
    """Per-head attention with wkv_b expanded: keys [q_absorb_w[h] c_kv ; k_pe], values
    out_absorb_w[h] c_kv; then concat heads and apply o_proj (no absorption)."""
    nh = inp["n_heads"]
    r = inp["kv_lora_rank"]
    scale = inp["softmax_scale"]
    rows = res["rows"][t][res["rows"][t] >= 0]
    slot = int(inp["slot_mapping"][t])
    keys = np.stack([res["stored_row"][t] if rr == slot else pool[rr] for rr in rows]) if len(rows) else np.zeros((0, r))
    q_nope, q_pe = trace["q_nope"][t], trace["q_pe"][t]
    outs = []
    for h in range(nh):
        k_nope = keys[:, :r] @ inp["q_absorb_w"][h].T  # [n, dn]
        v = keys[:, :r] @ inp["out_absorb_w"][h].T  # [n, dv]
        s = scale * (k_nope @ q_nope[h] + keys[:, r:] @ q_pe[h])
        p = np.exp(s - s.max())
        outs.append(p @ v / p.sum())
    return np.concatenate(outs) @ inp["o_proj_w"]


def _trace_q(inp):
    """q_nope / q_pe per token from the front-fold (pinned separately above)."""
    w = {k: inp[k] for k in ("input_norm_w", "wq_a", "q_norm_w", "wq_b", "wkv_a", "kv_norm_w", "q_absorb_w")}
    qn, qp = [], []
    for t in range(inp["hidden_states"].shape[0]):
        _, q_pe, q_nope, _ = oracle.front_fold(inp["hidden_states"][t], w, inp["cos"][t], inp["sin"][t],
                                               inp["n_heads"], inp["qk_nope_head_dim"],
                                               inp["qk_rope_head_dim"], inp["kv_lora_rank"], inp["norm_eps"])
        qn.append(q_nope)
        qp.append(q_pe)
    return {"q_nope": qn, "q_pe": qp}


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_absorbed_path_equals_explicit_wkv_b_mha(seed):
    inp, pool = _tiny_case(seed=seed)
    # make one token select its own (just written) position
    inp["gather_indices"][0, 3] = inp["positions"][0]
    res = _run(inp, pool)
    tr = _trace_q(inp)
    for t in range(2):
        ref = _explicit_mha_out(inp, res, tr, t, pool)
        np.testing.assert_allclose(res["out"][t], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_absorbed_path_equals_explicit_mha_on_tiny_workload():
    wl = CONFIGS[0]
    tin = make_inputs(wl)
    inp = oracle.to_f64_inputs(tin)
    pool = tin["kv_cache"].view(-1, wl.shape.kv_row_dim).double().numpy()
    res = _run(inp, pool)
    tr = _trace_q(inp)
    for t in range(wl.shape.n_tokens):
        ref = _explicit_mha_out(inp, res, tr, t, pool)
        np.testing.assert_allclose(res["out"][t], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_dense_selection_matches_torch_sdpa():
    """All prior positions selected, sorted, none masked: plain causal decode attention.
    Compared with torch's scaled_dot_product_attention in float64 on explicit heads."""
    T, P = 2, 12
    inp, pool = _tiny_case(seed=20, P=P, positions=[11, 11])
    inp["gather_indices"] = np.tile(np.arange(P), (T, 1))
    res = _run(inp, pool)
    assert res["mask"].all()
    tr = _trace_q(inp)
    r, nh = inp["kv_lora_rank"], inp["n_heads"]
    for t in range(T):
        rows = res["rows"][t]
        slot = int(inp["slot_mapping"][t])
        keys = np.stack([res["stored_row"][t] if rr == slot else pool[rr] for rr in rows])
        q = np.stack([np.concatenate([tr["q_nope"][t][h], tr["q_pe"][t][h]]) for h in range(nh)])
        k = np.stack([np.concatenate([keys[:, :r] @ inp["q_absorb_w"][h].T, keys[:, r:]], axis=1) for h in range(nh)])
        v = np.stack([keys[:, :r] @ inp["out_absorb_w"][h].T for h in range(nh)])
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            scale=inp["softmax_scale"])[0, :, 0, :].numpy()
        ref = o.reshape(-1) @ inp["o_proj_w"]
        np.testing.assert_allclose(res["out"][t], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_single_valid_entry_and_all_masked():
    inp, pool = _tiny_case(seed=30)
    pos0 = int(inp["positions"][0])
    gi = inp["gather_indices"]
    gi[0, :] = pos0 + 1  # every entry in the future ...
    gi[0, 5] = 2  # ... except one
    gi[1, :] = -3  # token 1: nothing valid
    res = _run(inp, pool)
    assert res["mask"][0].sum() == 1 and res["mask"][1].sum() == 0
    row = pool[res["rows"][0, 5]]
    r = inp["kv_lora_rank"]
    o_v = np.concatenate([inp["out_absorb_w"][h] @ row[:r] for h in range(inp["n_heads"])])
    np.testing.assert_allclose(res["out"][0], o_v @ inp["o_proj_w"], rtol=1e-12)
    assert np.array_equal(res["out"][1], np.zeros_like(res["out"][1]))


def test_self_row_is_read_after_write():
    """Selecting only the token's own position reads the row this step stored (bf16)."""
    inp, pool = _tiny_case(seed=31)
    gi = inp["gather_indices"]
    for t in range(2):
        gi[t, :] = -1
        gi[t, 0] = inp["positions"][t]
    res = _run(inp, pool)
    r = inp["kv_lora_rank"]
    for t in range(2):
        assert res["rows"][t, 0] == inp["slot_mapping"][t]
        row = res["stored_row"][t]
        assert np.array_equal(row, oracle.bf16_round(res["new_row"][t]))
        o_v = np.concatenate([inp["out_absorb_w"][h] @ row[:r] for h in range(inp["n_heads"])])
        np.testing.assert_allclose(res["out"][t], o_v @ inp["o_proj_w"], rtol=1e-12)


def test_zero_scale_averages_the_multiset():
    """softmax_scale = 0 gives uniform weights over valid entries, duplicates counted."""
    inp, pool = _tiny_case(seed=32, scale=0.0)
    gi = inp["gather_indices"]
    gi[0, 1] = gi[0, 0]
    gi[0, 2] = gi[0, 0]  # entry 0 now appears three times
    gi[0, 9] = 10**6  # masked
    res = _run(inp, pool, trace := {})
    r = inp["kv_lora_rank"]
    rows = res["rows"][0][res["rows"][0] >= 0]
    assert len(rows) == 9
    slot = int(inp["slot_mapping"][0])
    keys = np.stack([res["stored_row"][0] if rr == slot else pool[rr] for rr in rows])
    np.testing.assert_allclose(trace["o_lat"][0], np.tile(keys[:, :r].mean(0), (inp["n_heads"], 1)), rtol=1e-12)


def test_permutation_invariance():
    inp, pool = _tiny_case(seed=33)
    a = _run(inp, pool)["out"]
    rng = np.random.default_rng(0)
    inp["gather_indices"] = np.stack([rng.permutation(row) for row in inp["gather_indices"]])
    b = _run(inp, pool)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_doubling_every_entry_changes_nothing_but_one_duplicate_does():
    inp, pool = _tiny_case(seed=34)
    a = _run(inp, pool)["out"]
    inp2 = dict(inp)
    inp2["gather_indices"] = np.concatenate([inp["gather_indices"], inp["gather_indices"]], axis=1)
    b = _run(inp2, pool)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    inp3 = dict(inp)
    inp3["gather_indices"] = np.concatenate([inp["gather_indices"], inp["gather_indices"][:, :1]], axis=1)
    c = _run(inp3, pool)["out"]
    assert np.abs(c - a).max() > 1e-6  # a dedup would make this equal


def test_masked_rows_are_never_read():
    """NaN in every row a masked entry would resolve to, and future indices far past
    the block table, leave the output bit-identical."""
    inp, pool = _tiny_case(seed=35)
    bs = inp["kv_cache_block_size"]
    gi = inp["gather_indices"]
    gi[0, 0] = inp["positions"][0] + 1
    gi[1, 0] = inp["positions"][1] + 2
    a = _run(inp, pool)
    poisoned = pool.copy()
    for t in range(2):
        pos = int(inp["positions"][t])
        for g in range(pos + 1, inp["block_table"].shape[1] * bs):
            poisoned[inp["block_table"][t, g // bs] * bs + g % bs] = np.nan
    gi2 = gi.copy()
    gi2[0, 0] = 2**30
    gi2[1, 0] = 2**31 - 1
    inp2 = dict(inp, gather_indices=gi2)
    b = _run(inp2, poisoned)
    assert np.array_equal(a["out"], b["out"])


def test_cache_write_row_and_locality():
    """The stored row is the bf16 rounding of [RMSNorm(kv latent) | RoPE(k_pe)]; only
    slot_mapping rows are written (the oracle's overlay never touches the pool)."""
    wl = CONFIGS[0]
    tin = make_inputs(wl)
    inp = oracle.to_f64_inputs(tin)
    pool = tin["kv_cache"].view(-1, wl.shape.kv_row_dim).double().numpy()
    before = pool.copy()
    res = _run(inp, pool)
    assert np.array_equal(before, pool)
    r = wl.shape.kv_lora_rank
    for t in range(wl.shape.n_tokens):
        xh = oracle.rms_norm(inp["hidden_states"][t], inp["input_norm_w"], 1e-6)
        kv = xh @ inp["wkv_a"]
        ref = np.concatenate([oracle.rms_norm(kv[:r], inp["kv_norm_w"], 1e-6),
                              oracle.rope_interleaved(kv[r:], inp["cos"][t], inp["sin"][t])])
        np.testing.assert_allclose(res["new_row"][t], ref, rtol=1e-13)
        assert np.array_equal(res["stored_row"][t],
                              torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).double().numpy())
