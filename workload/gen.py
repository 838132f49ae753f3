"""Seeded synthetic inputs for one MLA gather-decode step.

Tensor names, shapes and index semantics follow the parameter list of the
"MLA Attention Block Gather Decode Kernel API Reference" page (section
"API Reference").  Value distributions follow the workload recipes stated for
the five benchmark shapes (tiny, DeepSeek-V3.2 slice, batch 32, full-head 64,
large-batch long-context 128).

Two kinds of random streams are used:

* every dense tensor except the cache pool draws from its own
  ``numpy.random.PCG64`` stream seeded by ``SeedSequence([seed, tag])``, so a
  tensor does not depend on the order in which the others are drawn;
* the paged cache pool (up to 19.3 GB) is defined element by element by a
  counter-based generator: the e-th output of SplitMix64 (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) with
  a seed-derived state, whose top 16 bits index a 65536-entry table of
  standard-normal quantiles rounded to bf16.  The same integer code runs on
  any torch device, so the GPU can fill the pool in place while the oracle
  regenerates exactly the rows it needs on the host.

Nothing here computes any part of the step: no norms, projections, rotary
embedding, index resolution or attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from functools import lru_cache
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# ----------------------------------------------------------------------------
# shapes and workload recipes
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class MlaShape:
    """Dimensions of one step.  Names follow the page's parameters."""

    n_tokens: int
    hidden: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    n_heads: int
    block_size: int
    max_blocks_per_seq: int
    n_prior: int
    softmax_scale: float
    norm_eps: float = 1e-6

    @property
    def kv_row_dim(self) -> int:
        # one cache row = [latent (kv_lora_rank) | rotary key (qk_rope_head_dim)]
        return self.kv_lora_rank + self.qk_rope_head_dim

    @property
    def qk_head_dim(self) -> int:
        return self.qk_nope_head_dim + self.qk_rope_head_dim

    @property
    def qk_packed_dim(self) -> int:
        return self.n_heads * self.qk_head_dim

    @property
    def n_blocks(self) -> int:
        # every sequence owns max_blocks_per_seq distinct blocks of one shared pool
        return self.n_tokens * self.max_blocks_per_seq


@dataclass(frozen=True)
class Workload:
    """A named shape plus the recipe its synthetic inputs are drawn from."""

    name: str
    shape: MlaShape
    seed: int
    # either explicit contexts (one per token) or an inclusive uniform range
    contexts: Optional[Tuple[int, ...]] = None
    context_range: Optional[Tuple[int, int]] = None
    n_duplicates: int = 0  # entries that repeat an already selected position
    n_future: int = 0  # entries past the token's position (causally masked)
    description: str = ""
    # tokens per sequence in the step (speculative / multi-token decode): the
    # tokens of a sequence sit at its last positions, share its block-table
    # row (token_seq), and each selects every other one of them
    tokens_per_seq: int = 1

    def with_tokens(self, n_tokens: int) -> "Workload":
        """Same recipe with fewer tokens (used by tests to sample a big shape)."""
        sh = replace(self.shape, n_tokens=n_tokens)
        ctx = self.contexts[:n_tokens] if self.contexts is not None else None
        return replace(self, shape=sh, contexts=ctx)


_DS32 = dict(hidden=7168, q_lora_rank=1536, kv_lora_rank=512, qk_nope_head_dim=128,
             qk_rope_head_dim=64, v_head_dim=128, block_size=64, n_prior=2048,
             softmax_scale=1.0 / math.sqrt(192.0), norm_eps=1e-6)

CONFIGS: List[Workload] = [
    Workload(
        name="tiny",
        shape=MlaShape(n_tokens=2, hidden=256, q_lora_rank=64, kv_lora_rank=64,
                       qk_nope_head_dim=32, qk_rope_head_dim=16, v_head_dim=32, n_heads=4,
                       block_size=16, max_blocks_per_seq=8, n_prior=32,
                       softmax_scale=1.0 / math.sqrt(48.0), norm_eps=1e-6),
        seed=1000, contexts=(41, 101), n_duplicates=3, n_future=2,
        description="T=2, H=256, nh=4, positions 40 and 100, 27 distinct + 3 dup + 2 future",
    ),
    Workload(
        name="ds32_slice",
        shape=MlaShape(n_tokens=1, n_heads=16, max_blocks_per_seq=128, **_DS32),
        seed=1001, contexts=(8192,),
        description="T=1, nh=16, context 8192, 2048 distinct prior positions",
    ),
    Workload(
        name="batch32",
        shape=MlaShape(n_tokens=32, n_heads=16, max_blocks_per_seq=512, **_DS32),
        seed=1002, context_range=(4096, 32768),
        description="T=32, nh=16, contexts U[4096,32768]",
    ),
    Workload(
        name="fullhead64",
        shape=MlaShape(n_tokens=64, n_heads=128, max_blocks_per_seq=1024, **_DS32),
        seed=1003, context_range=(16384, 65536),
        description="T=64, nh=128, contexts U[16384,65536]",
    ),
    Workload(
        name="large128",
        shape=MlaShape(n_tokens=128, n_heads=128, max_blocks_per_seq=2048, **_DS32),
        seed=1004, context_range=(65536, 131072), n_duplicates=205,
        description="T=128, nh=128, contexts U[65536,131072], 19.3 GB pool, 10% duplicates",
    ),
]


def config_by_name(name: str) -> Workload:
    for w in CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------
# per-tensor PCG64 streams
# ----------------------------------------------------------------------------

_TAGS: Dict[str, int] = {
    "hidden_states": 1, "input_norm_w": 2, "wq_a": 3, "q_norm_w": 4, "wq_b": 5,
    "wkv_a": 6, "kv_norm_w": 7, "q_absorb_w": 8, "out_absorb_w": 9, "o_proj_w": 10,
    "contexts": 11, "block_table": 12, "gather_indices": 13, "kv_pool": 14,
    "router_hidden": 21, "router_gamma": 22, "router_weights": 23, "router_bias": 24,
}


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[name]])))


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)


def _normal_bf16(seed: int, name: str, shape: Sequence[int], std: float) -> torch.Tensor:
    z = _rng(seed, name).standard_normal(size=tuple(shape))
    return _bf16(z * std)


# ----------------------------------------------------------------------------
# counter-based pool generator (SplitMix64 -> normal quantile table)
# ----------------------------------------------------------------------------

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_U64 = (1 << 64) - 1


def _as_i64(x: int) -> int:
    x &= _U64
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr_t(z: torch.Tensor, k: int) -> torch.Tensor:
    # logical right shift of int64 bit patterns (torch's >> is arithmetic)
    return torch.bitwise_and(torch.bitwise_right_shift(z, k), (1 << (64 - k)) - 1)


def splitmix64_torch(state: int, idx: torch.Tensor) -> torch.Tensor:
    """Output number ``idx`` (0-based) of SplitMix64 started at ``state``.

    ``idx`` is an int64 tensor; the result holds the 64-bit outputs as int64 bit
    patterns.  int64 multiplication wraps modulo 2^64 on every torch device, so
    the bits equal the unsigned reference computation.
    """
    z = (idx + 1) * _as_i64(_GAMMA) + _as_i64(state)
    z = torch.bitwise_xor(z, _lsr_t(z, 30)) * _as_i64(_M1)
    z = torch.bitwise_xor(z, _lsr_t(z, 27)) * _as_i64(_M2)
    return torch.bitwise_xor(z, _lsr_t(z, 31))


def splitmix64_np(state: int, idx: np.ndarray) -> np.ndarray:
    """Unsigned numpy version of :func:`splitmix64_torch` (cross-check only)."""
    with np.errstate(over="ignore"):
        z = (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(_GAMMA) + np.uint64(state & _U64)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


@lru_cache(maxsize=1)
def _normal_table_cpu() -> torch.Tensor:
    from scipy.special import ndtri

    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return _bf16(ndtri(u))


def _normal_table(device) -> torch.Tensor:
    return _normal_table_cpu().to(device)


def _pool_state(seed: int) -> int:
    return ((seed & 0xFFFFFFFF) << 32) | _TAGS["kv_pool"]


def _pool_values(seed: int, first_elem: int, n_elem: int, device) -> torch.Tensor:
    idx = torch.arange(first_elem, first_elem + n_elem, dtype=torch.int64, device=device)
    top16 = _lsr_t(splitmix64_torch(_pool_state(seed), idx), 48)
    return _normal_table(device)[top16]


def fill_pool_(wl: Workload, pool: torch.Tensor, chunk_rows: int = 1 << 18) -> torch.Tensor:
    """Fill a ``[n_blocks, 1, block_size, kv_row_dim]`` bf16 pool in place, on its device."""
    sh = wl.shape
    n_rows = sh.n_blocks * sh.block_size
    flat = pool.view(n_rows, sh.kv_row_dim)
    for r0 in range(0, n_rows, chunk_rows):
        r1 = min(n_rows, r0 + chunk_rows)
        vals = _pool_values(wl.seed, r0 * sh.kv_row_dim, (r1 - r0) * sh.kv_row_dim, pool.device)
        flat[r0:r1].copy_(vals.view(r1 - r0, sh.kv_row_dim))
    return pool


def pool_rows(wl: Workload, rows: np.ndarray) -> torch.Tensor:
    """Regenerate the listed flat pool rows on the host: bf16 ``[len(rows), kv_row_dim]``.

    Rows are the original pool content, before any step writes into it.
    """
    kv = wl.shape.kv_row_dim
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    elem = (rows[:, None] * kv + np.arange(kv, dtype=np.int64)[None, :]).reshape(-1)
    idx = torch.from_numpy(elem)
    top16 = _lsr_t(splitmix64_torch(_pool_state(wl.seed), idx), 48)
    return _normal_table_cpu()[top16].view(len(rows), kv)


# ----------------------------------------------------------------------------
# the full input set
# ----------------------------------------------------------------------------


def _contexts(wl: Workload) -> np.ndarray:
    T = wl.shape.n_tokens
    if wl.contexts is not None:
        c = np.asarray(wl.contexts[:T], dtype=np.int64)
        assert len(c) == T
        return c
    lo, hi = wl.context_range
    return _rng(wl.seed, "contexts").integers(lo, hi, size=T, endpoint=True)


def _gather_indices(wl: Workload, positions: np.ndarray, step_positions=None) -> np.ndarray:
    """step_positions[t]: positions of the other tokens of t's sequence in this
    step, each selected once (earlier ones valid, later ones masked)."""
    sh = wl.shape
    P = sh.n_prior
    seq_cap = sh.max_blocks_per_seq * sh.block_size  # positions a block-table row can address
    rng = _rng(wl.seed, "gather_indices")
    out = np.empty((sh.n_tokens, P), dtype=np.int64)
    for t, pos in enumerate(positions.tolist()):
        forced = np.asarray([] if step_positions is None else step_positions[t], dtype=np.int64)
        n_dist = P - wl.n_duplicates - wl.n_future - len(forced)
        early = forced[forced <= pos]
        n_avail = pos + 1
        take = min(n_dist, n_avail - len(early))
        pool = np.setdiff1d(np.arange(n_avail), early) if len(early) else None
        distinct = (rng.choice(pool, size=take, replace=False) if pool is not None
                    else rng.choice(n_avail, size=take, replace=False))
        distinct = np.concatenate([distinct, early]).astype(np.int64)
        n_fut = wl.n_future + (n_dist - take)  # short sequences pad with masked future positions
        dups = rng.choice(distinct, size=wl.n_duplicates, replace=False) if wl.n_duplicates else np.empty(0, np.int64)
        if n_fut:
            assert pos + 1 <= seq_cap - 1, "no room for future positions"
            fut = rng.integers(pos + 1, seq_cap - 1, size=n_fut, endpoint=True)
        else:
            fut = np.empty(0, np.int64)
        row = np.concatenate([distinct, dups, fut, forced[forced > pos]]).astype(np.int64)
        rng.shuffle(row)
        out[t] = row
    return out


def make_inputs(wl: Workload, device="cpu", with_pool: bool = True,
                pool_device=None) -> Dict[str, object]:
    """Draw every tensor of one step.

    Returns a dict keyed by the page's parameter names (plus the scalar
    parameters).  Gammas are ``[1, n]`` fp32, index tensors int32, everything
    else bf16.  ``kv_cache`` is allocated and filled on ``pool_device``
    (default: ``device``) unless ``with_pool`` is false.
    """
    sh = wl.shape
    T, H, Q, r = sh.n_tokens, sh.hidden, sh.q_lora_rank, sh.kv_lora_rank
    dn, dr, dv, nh = sh.qk_nope_head_dim, sh.qk_rope_head_dim, sh.v_head_dim, sh.n_heads
    bs, MB = sh.block_size, sh.max_blocks_per_seq
    kvr = sh.kv_row_dim
    s = wl.seed

    def gamma(name, n):
        g = 1.0 + 0.1 * _rng(s, name).standard_normal(size=(1, n))
        return torch.from_numpy(g).to(torch.float32)

    out: Dict[str, object] = {}
    out["hidden_states"] = _normal_bf16(s, "hidden_states", (T, H), 1.0)
    out["input_norm_w"] = gamma("input_norm_w", H)
    out["wq_a"] = _normal_bf16(s, "wq_a", (H, Q), 1.0 / math.sqrt(H))
    out["q_norm_w"] = gamma("q_norm_w", Q)
    out["wq_b"] = _normal_bf16(s, "wq_b", (Q, sh.qk_packed_dim), 1.0 / math.sqrt(Q))
    out["wkv_a"] = _normal_bf16(s, "wkv_a", (H, kvr), 1.0 / math.sqrt(H))
    out["kv_norm_w"] = gamma("kv_norm_w", r)
    # both halves of wkv_b take the latent (width kv_lora_rank) as their input
    out["q_absorb_w"] = _normal_bf16(s, "q_absorb_w", (nh, dn, r), 1.0 / math.sqrt(r))
    out["out_absorb_w"] = _normal_bf16(s, "out_absorb_w", (nh, dv, r), 1.0 / math.sqrt(r))
    out["o_proj_w"] = _normal_bf16(s, "o_proj_w", (nh * dv, H), 1.0 / math.sqrt(nh * dv))

    ctx = _contexts(wl)
    positions = ctx - 1  # the current token is the last position of its context
    assert np.all(positions < MB * bs), "context longer than the block table can address"
    perm = _rng(s, "block_table").permutation(sh.n_blocks).astype(np.int64)
    block_table = perm.reshape(T, MB)
    k = wl.tokens_per_seq
    step_positions = None
    if k > 1:
        # token j of sequence q = t // k sits k - 1 - j positions before the
        # end of that sequence's context; the table has one row per sequence
        assert T % k == 0, "tokens_per_seq must divide n_tokens"
        seq = np.arange(T) // k
        positions = ctx[seq * k + k - 1] - 1 - (k - 1 - np.arange(T) % k)
        assert np.all(positions >= 0)
        block_table = block_table[: T // k]
        out["token_seq"] = torch.from_numpy(seq.astype(np.int32))
        step_positions = [[int(positions[u]) for u in range(q * k, q * k + k) if u != t]
                          for t, q in enumerate(seq.tolist())]
    else:
        seq = np.arange(T)
    # this token's own key lives at logical position `pos` of its sequence:
    # physical block block_table[seq, pos // bs], offset pos % bs in that block
    slot = block_table[seq, positions // bs] * bs + positions % bs
    gi = _gather_indices(wl, positions, step_positions)

    # rotary tables evaluated at the token's position, theta_i = pos * 10000^(-2i/dr)
    i = np.arange(dr // 2, dtype=np.float64)
    ang = positions.astype(np.float64)[:, None] * np.power(10000.0, -2.0 * i / dr)[None, :]
    out["cos"] = torch.from_numpy(np.cos(ang)).to(torch.float32)
    out["sin"] = torch.from_numpy(np.sin(ang)).to(torch.float32)

    out["slot_mapping"] = torch.from_numpy(slot.astype(np.int32))
    out["block_table"] = torch.from_numpy(block_table.astype(np.int32))
    out["positions"] = torch.from_numpy(positions.astype(np.int32))
    out["gather_indices"] = torch.from_numpy(gi.astype(np.int32))

    out["n_heads"] = nh
    out["qk_nope_head_dim"] = dn
    out["qk_rope_head_dim"] = dr
    out["kv_lora_rank"] = r
    out["softmax_scale"] = float(sh.softmax_scale)
    out["norm_eps"] = float(sh.norm_eps)

    dev = torch.device(device)
    for k, v in list(out.items()):
        if isinstance(v, torch.Tensor):
            out[k] = v.to(dev)
    if with_pool:
        pdev = torch.device(pool_device) if pool_device is not None else dev
        pool = torch.empty((sh.n_blocks, 1, bs, kvr), dtype=torch.bfloat16, device=pdev)
        out["kv_cache"] = fill_pool_(wl, pool)
    return out


def to_device(wl: Workload, inp: Dict[str, object], device="cuda") -> Dict[str, object]:
    """Copy the tensors of a host input set to ``device``; the cache pool is
    copied if the set holds one, else allocated and filled there in place."""
    sh = wl.shape
    g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items() if k != "kv_cache"}
    if "kv_cache" in inp:
        g["kv_cache"] = inp["kv_cache"].to(device)
    else:
        pool = torch.empty((sh.n_blocks, 1, sh.block_size, sh.kv_row_dim), dtype=torch.bfloat16, device=device)
        g["kv_cache"] = fill_pool_(wl, pool)
    return g


# ----------------------------------------------------------------------------
# the fused RMSNorm + router top-K (the MoE block's first step)
# ----------------------------------------------------------------------------

# (n_tokens, hidden, n_experts, top_k): DeepSeek-V3-sized routers at one and at
# the page's largest token count
ROUTER_CONFIGS = {
    "router_t1": (1, 7168, 256, 8),
    "router_t128": (128, 7168, 256, 8),
}


def make_router_inputs(n_tokens: int, hidden: int, n_experts: int, seed: int, with_bias: bool = True,
                       dtype=torch.bfloat16):
    """hidden_states [T, H] ~ N(0, 1), gamma [H] ~ 1 + 0.1 N, router weights
    [H, E] ~ N(0, 1/H) (logits of unit scale), all three in `dtype` (bf16 or
    fp16, the page's two input types; the same draws either way), bias [E]
    fp32 ~ 0.1 N."""
    def cast(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.float32).to(dtype)

    out = {
        "hidden_states": cast(_rng(seed, "router_hidden").standard_normal(size=(n_tokens, hidden))),
        "gamma": cast(1.0 + 0.1 * _rng(seed, "router_gamma").standard_normal(size=(hidden,))),
        "router_weights": cast(_rng(seed, "router_weights").standard_normal(size=(hidden, n_experts))
                               * (1.0 / math.sqrt(hidden))),
        "router_bias": None,
    }
    if with_bias:
        b = 0.1 * _rng(seed, "router_bias").standard_normal(size=(n_experts,))
        out["router_bias"] = torch.from_numpy(b).to(torch.float32)
    return out
