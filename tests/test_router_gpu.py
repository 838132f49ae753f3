"""GPU parity of the fused RMSNorm + router top-K against the fp64 router oracle.

Bars: normalised states, and the affinities of the selected experts (bf16),
within max |err| <= 2e-2 * RMS of the oracle's values; unselected affinities
exactly zero; the selected experts are the oracle's top-K up to ranking ties
within TOL_LOGIT of each other (fp32 against fp64 logits): every selected
logit is at least every unselected one minus TOL_LOGIT and the order is
descending within it, and where the oracle's ranking has no such near-tie the
indices are bit-exact.  Affinities are checked at the experts the GPU chose.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import router_oracle as ro
from sparse_gather_mla_amd.router import rmsnorm_router_topk
from tests.harness import within_tol
from workload import ROUTER_CONFIGS, make_router_inputs

pytestmark = pytest.mark.gpu
TOL_LOGIT = 1e-3


def _f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def _check(T, H, E, K, act, with_bias, seed, zero_weights=False, dtype=torch.bfloat16):
    print(f"[router] T={T} H={H} E={E} K={K} act={act} bias={with_bias} dtype={dtype}", flush=True)
    sys.stdout.flush()
    inp = make_router_inputs(T, H, E, seed, with_bias, dtype=dtype)
    if zero_weights:
        inp["router_weights"].zero_()
    g = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    normed, idx, aff = rmsnorm_router_topk(g["hidden_states"], g["gamma"], g["router_weights"], g["router_bias"],
                                           1e-6, K, act)
    torch.cuda.synchronize()
    x, gam, w = _f64(inp["hidden_states"]), _f64(inp["gamma"]), _f64(inp["router_weights"])
    b = _f64(inp["router_bias"]) if with_bias else None
    a = ro.SIGMOID if act == "sigmoid" else ro.SOFTMAX
    x_hat, ref_idx, _ = ro.rmsnorm_router_topk(x, gam, w, b, 1e-6, K, a)
    z = ro.router_logits(x_hat, w, b)
    assert normed.dtype == dtype and aff.dtype == torch.bfloat16
    ok, err, bound = within_tol(_f64(normed), x_hat)
    assert ok, ("normed", err, bound)
    if dtype == torch.float16:  # fp16 keeps 3 more mantissa bits than bf16: a tighter floor holds
        assert np.max(np.abs(_f64(normed) - x_hat)) <= 2.0 ** -10 * np.max(np.abs(x_hat)), "normed (fp16 rounding)"
    got = idx.cpu().numpy().astype(np.int64)
    ref_aff = np.zeros((T, E))
    n_exact = 0
    for t in range(T):
        sel = got[t]
        assert len(set(sel.tolist())) == K and sel.min() >= 0 and sel.max() < E
        zt = z[t]
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            assert zt[sel].min() >= zt[rest].max() - TOL_LOGIT
        assert np.all(np.diff(zt[sel]) <= TOL_LOGIT)
        srt = np.sort(zt)[::-1]
        if np.all(np.abs(np.diff(srt[:K + 1])) > TOL_LOGIT):  # no near-tie in the ranking
            assert np.array_equal(sel, ref_idx[t])
            n_exact += 1
        ref_aff[t, sel] = ro.activate_selected(zt[sel], a)
    got_aff = _f64(aff)
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, got, True, axis=1)
    assert np.all(got_aff[~mask] == 0)  # unselected experts: exact zeros
    # selected: the bar is relative to the selected values (the zeros would shrink an RMS over the whole row)
    ok, err, bound = within_tol(got_aff[mask], ref_aff[mask])
    assert ok, ("affinities", err, bound)
    print(f"[router] ok: {n_exact}/{T} tokens bit-exact rankings, affinity err {err:.2e} (bound {bound:.2e})",
          flush=True)
    return got, got_aff


@pytest.mark.parametrize("name,act", [("router_t1", "sigmoid"), ("router_t128", "softmax")])
def test_router_full_size(name, act):
    T, H, E, K = ROUTER_CONFIGS[name]
    _check(T, H, E, K, act, True, seed=31)


@pytest.mark.parametrize("T,H,E,K,act,bias", [
    (8, 7168, 256, 8, "softmax", False),   # one full token pass
    (37, 1152, 72, 5, "sigmoid", True),    # ragged: 4 passes + 5 tokens, a 64 + 8 expert split
    (3, 256, 64, 32, "softmax", True),     # the largest top_k
    (128, 128, 8, 8, "sigmoid", False),    # every expert selected, the smallest hidden
    (9, 7168, 256, 8, "sigmoid", True),    # the fewest tokens on the matrix cores: one padded token block
    (65, 384, 1000, 16, "softmax", True),  # three token blocks, eight expert tiles with a 104-expert tail
])
def test_router_ragged_and_limits(T, H, E, K, act, bias):
    _check(T, H, E, K, act, bias, seed=41 + T)


@pytest.mark.parametrize("T,H,E,K,act", [
    (1, 7168, 256, 8, "sigmoid"),   # router_t1 in fp16
    (37, 1152, 72, 5, "softmax"),   # ragged, fp16
])
def test_router_fp16_inputs(T, H, E, K, act):
    _check(T, H, E, K, act, True, seed=61 + T, dtype=torch.float16)


def test_router_largest_expert_count():
    """n_experts = 1024 (16 logits per lane of the top-K wave, 16 expert tiles)
    with the largest top_k."""
    _check(3, 256, 1024, 32, "sigmoid", True, seed=71)


def test_router_exact_ties_pick_lower_experts():
    """Zero router weights and no bias: every logit is 0, so the first K experts
    are chosen in index order, each with sigmoid(0) = 1/2."""
    got, aff = _check(4, 256, 32, 6, "sigmoid", False, seed=5, zero_weights=True)
    assert np.array_equal(got, np.tile(np.arange(6), (4, 1)))
    assert np.all(aff[:, :6] == 0.5) and np.all(aff[:, 6:] == 0)


@pytest.mark.parametrize("H,E,K,act", [
    (1152, 72, 5, "softmax"),   # a 64 + 8 expert split
    (256, 1024, 32, "sigmoid"),  # the top-K wave (more than 256 experts)
])
def test_router_one_token_shapes(H, E, K, act):
    """One token runs as a single launch whose last workgroup selects."""
    _check(1, H, E, K, act, True, seed=81 + E)


def test_router_one_token_repeats_on_one_workspace():
    """The single-token launch counts its workgroups in the workspace and the
    last one resets the counter: three calls on one workspace give the same
    bits, agree with the oracle, and leave the counter at zero."""
    from sparse_gather_mla_amd.router import workspace_size

    T, H, E, K = ROUTER_CONFIGS["router_t1"]
    _check(T, H, E, K, "sigmoid", True, seed=91)
    inp = make_router_inputs(T, H, E, 91, True)
    g = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    ws = torch.zeros(workspace_size(T, H, E), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        normed, idx, aff = rmsnorm_router_topk(g["hidden_states"], g["gamma"], g["router_weights"], g["router_bias"],
                                               1e-6, K, "sigmoid", workspace=ws)
        torch.cuda.synchronize()
        outs.append((normed.clone(), idx.clone(), aff.clone()))
        assert int(ws[:4].view(torch.int32).item()) == 0
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(o, outs[0]))
