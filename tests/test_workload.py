"""The seeded synthetic inputs: determinism, recipe invariants, pool regeneration."""
import numpy as np
import pytest
import torch

from workload import CONFIGS, make_inputs, pool_rows, splitmix64_np, splitmix64_torch
from workload.gen import fill_pool_


def test_splitmix64_reference_outputs_and_torch_agrees_with_numpy():
    # published first outputs of SplitMix64 seeded with 0
    got = splitmix64_np(0, np.arange(3))
    assert [hex(int(v)) for v in got] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]
    idx = np.array([0, 1, 17, 2**33 + 5, 2**62 + 3, 9_663_676_415], dtype=np.int64)
    for state in (0, 12345, (1004 << 32) | 14, 2**64 - 1):
        a = splitmix64_np(state, idx)
        b = splitmix64_torch(state, torch.from_numpy(idx)).numpy().view(np.uint64)
        assert np.array_equal(a, b)


def test_inputs_are_deterministic():
    a = make_inputs(CONFIGS[0])
    b = make_inputs(CONFIGS[0])
    for k, v in a.items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(v, b[k]), k
        else:
            assert v == b[k]


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_recipe_invariants(idx):
    wl = CONFIGS[idx]
    sh = wl.shape
    inp = make_inputs(wl, with_pool=False)
    T, P, bs, MB = sh.n_tokens, sh.n_prior, sh.block_size, sh.max_blocks_per_seq
    bt = inp["block_table"].numpy().astype(np.int64)
    pos = inp["positions"].numpy().astype(np.int64)
    gi = inp["gather_indices"].numpy().astype(np.int64)
    slot = inp["slot_mapping"].numpy().astype(np.int64)
    assert bt.shape == (T, MB) and np.array_equal(np.sort(bt.reshape(-1)), np.arange(T * MB))
    assert gi.shape == (T, P)
    assert len(set(slot.tolist())) == T
    assert np.all(slot // bs == bt[np.arange(T), pos // bs]) and np.all(slot % bs == pos % bs)
    if wl.contexts is not None:
        assert list(pos + 1) == list(wl.contexts[:T])
    else:
        lo, hi = wl.context_range
        assert np.all((pos + 1 >= lo) & (pos + 1 <= hi))
    for t in range(T):
        valid = gi[t][(gi[t] >= 0) & (gi[t] <= pos[t])]
        fut = gi[t][gi[t] > pos[t]]
        assert len(fut) == wl.n_future
        assert np.all(fut < MB * bs)
        assert len(valid) - len(np.unique(valid)) == wl.n_duplicates
        assert not np.array_equal(gi[t], np.sort(gi[t]))  # unsorted
    assert inp["cos"].shape == (T, sh.qk_rope_head_dim // 2)
    assert inp["input_norm_w"].shape == (1, sh.hidden) and inp["input_norm_w"].dtype == torch.float32


def test_weight_distributions():
    inp = make_inputs(CONFIGS[1], with_pool=False)
    for name, fan_in in (("wq_a", 7168), ("wq_b", 1536), ("wkv_a", 7168), ("q_absorb_w", 512),
                         ("out_absorb_w", 512), ("o_proj_w", 2048)):
        w = inp[name].float()
        assert w.dtype == torch.float32 and abs(w.std().item() * fan_in ** 0.5 - 1) < 0.02, name
    g = inp["q_norm_w"]
    assert abs(g.mean().item() - 1) < 0.01 and abs(g.std().item() - 0.1) < 0.01


def test_pool_regeneration_matches_in_place_fill():
    wl = CONFIGS[0]
    sh = wl.shape
    pool = torch.empty((sh.n_blocks, 1, sh.block_size, sh.kv_row_dim), dtype=torch.bfloat16)
    fill_pool_(wl, pool, chunk_rows=37)  # chunking must not matter
    flat = pool.view(-1, sh.kv_row_dim)
    rows = np.array([0, 5, 255, 17, 5])
    assert torch.equal(pool_rows(wl, rows), flat[rows])
    v = flat.float()
    assert abs(v.mean().item()) < 0.05 and abs(v.std().item() - 1) < 0.05
