"""Plain fp64 CPU oracle for one MLA gather-decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module; the GPU library
never calls it and shares no code with it.

What it computes is read off the "MLA Attention Block Gather Decode Kernel API
Reference" page (awsdocs-neuron, nkilib experimental deepseek_v32): the opening
description, the "API Reference" parameter list, and the "Notes" and
"Dimensions" sections.  The page prints no numeric example, so every value
here is pinned by the checks in tests/test_oracle_pins.py (closed forms,
library routines, invariants and brute force), not by printed numbers.

Everything is evaluated per token, in float64, in the order the page lists
the operations, with no tiling, splitting or online softmax.  Inputs are the
exact bf16 / fp32 / int32 values widened to float64.  The only rounding
modelled is the bf16 storage of the cache row this step writes (the page says
the core reads back what the front-fold wrote into the cache).

Readings taken where the page is silent:
  * weights are used as ``y = x @ W`` with the printed ``[in, out]`` shapes;
  * ``wq_b`` columns are head-major, each head ``[q_nope | q_pe]``;
  * a cache row is ``[kv latent (kv_lora_rank) | rotary key (qk_rope_head_dim)]``;
  * RMSNorm is ``x / sqrt(mean(x^2) + eps) * gamma``;
  * interleaved RoPE rotates adjacent pairs (2i, 2i+1) by angle i;
  * a selected position g is valid iff 0 <= g <= positions[t]; masked entries
    touch neither the block table nor the cache;
  * selected positions form a multiset (duplicates are separate softmax terms);
  * a token with no valid entry gets a zero latent output;
  * the output is this rank's partial o-projection (no residual, no reduction).
"""
from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# elementary pieces
# ---------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  Used only
    for the cache row the step stores (the ``kv_cache`` parameter of "API
    Reference": the cache is updated in place and later gathered from).
    """
    x = np.asarray(x, dtype=F64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    m, e = np.frexp(x[fin])  # x = m * 2^e, 0.5 <= |m| < 1
    q_exp = np.maximum(e - 8, -133)  # quantum of 8 significant bits; subnormal floor 2^-133
    y = np.ldexp(np.rint(np.ldexp(x[fin], -q_exp)), q_exp)  # np.rint: half to even
    max_bf16 = np.ldexp(F64(255.0), 120)  # (2 - 2^-7) * 2^127
    y = np.where(np.abs(y) > max_bf16, np.copysign(np.inf, y), y)
    out[fin] = y
    return out


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: ``x / sqrt(mean(x^2) + eps) * gamma``.

    The page gives fp32 RMSNorm scales for three places (the layer input, the
    query latent and the KV latent) and a single ``norm_eps`` that all three
    norms share ("API Reference": ``input_norm_w``, ``q_norm_w``,
    ``kv_norm_w``, ``norm_eps``).
    """
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + F64(eps)) * np.asarray(gamma, dtype=F64).reshape(-1)


def rope_interleaved(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Interleaved rotary embedding of the last axis.

    ``cos``/``sin`` have ``qk_rope_dim // 2`` entries ("API Reference": ``cos``,
    ``sin``); pair i is the adjacent pair (2i, 2i+1), rotated in place:
    ``(x0, x1) -> (x0*c - x1*s, x0*s + x1*c)``.
    """
    x = np.asarray(x, dtype=F64)
    c = np.asarray(cos, dtype=F64)
    s = np.asarray(sin, dtype=F64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def resolve_row(g: int, position: int, block_table_row: np.ndarray, block_size: int) -> int:
    """Index build for one selected position ("API Reference": ``block_table``,
    ``positions``, ``gather_indices``).

    A selected absolute position g is causally valid iff ``0 <= g <= position``;
    a valid position lives in logical block ``g // block_size`` of the
    sequence, which the block table maps to a physical block, at offset
    ``g % block_size``.  The flat cache row is ``physical * block_size +
    offset``.  Masked positions return -1 and read nothing.
    """
    if g < 0 or g > position:
        return -1
    phys = int(block_table_row[g // block_size])
    return phys * block_size + (g % block_size)


# ---------------------------------------------------------------------------
# the two halves of the block
# ---------------------------------------------------------------------------

def front_fold(x_t: np.ndarray, w: Dict[str, np.ndarray], cos_t: np.ndarray, sin_t: np.ndarray,
               n_heads: int, dn: int, dr: int, r: int, eps: float):
    """QKV front-fold for one token.

    Follows the order of the page's parameter list: input RMSNorm, ``wq_a``
    down-projection, query-latent RMSNorm, ``wq_b`` up-projection (every
    head's ``[q_nope | q_pe]``), ``wkv_a`` down-projection to one cache row,
    KV-latent RMSNorm of its first ``kv_lora_rank`` entries, interleaved RoPE
    on ``q_pe`` and on the row's rotary part, and the absorption of each
    head's nope query into the latent with ``q_absorb_w``.

    Returns ``(q_lat [nh, r], q_pe [nh, dr], q_nope [nh, dn], new_row [r + dr])``.
    """
    xh = rms_norm(x_t, w["input_norm_w"], eps)
    q_a = xh @ w["wq_a"]
    c_q = rms_norm(q_a, w["q_norm_w"], eps)
    q = (c_q @ w["wq_b"]).reshape(n_heads, dn + dr)
    q_nope = q[:, :dn]
    q_pe = rope_interleaved(q[:, dn:], cos_t, sin_t)

    kv = xh @ w["wkv_a"]
    c_kv = rms_norm(kv[:r], w["kv_norm_w"], eps)
    k_pe = rope_interleaved(kv[r:], cos_t, sin_t)
    new_row = np.concatenate([c_kv, k_pe])

    q_lat = np.empty((n_heads, r), dtype=F64)
    for h in range(n_heads):
        q_lat[h] = q_nope[h] @ w["q_absorb_w"][h]  # [dn] @ [dn, r]
    return q_lat, q_pe, q_nope, new_row


def attention_core(q_lat: np.ndarray, q_pe: np.ndarray, keys: np.ndarray, scale: float,
                   r: int) -> np.ndarray:
    """Softmax attention of every head over the gathered rows, in latent space.

    ``keys`` holds one gathered row per valid selected entry (duplicates
    included).  Score = ``softmax_scale * (q_lat . row[:r] + q_pe . row[r:])``
    ("API Reference": ``softmax_scale``, ``kv_lora_rank``); the value is the
    row's latent part, the width ``out_absorb_w`` maps back out.  An empty set
    gives a zero output.  Returns ``o_lat [nh, r]``.
    """
    nh = q_lat.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((nh, r), dtype=F64)
    s = F64(scale) * (q_lat @ keys[:, :r].T + q_pe @ keys[:, r:].T)  # [nh, n]
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ keys[:, :r]) / np.sum(p, axis=1, keepdims=True)


def output_projection(o_lat: np.ndarray, out_absorb_w: np.ndarray, o_proj_w: np.ndarray) -> np.ndarray:
    """``out_absorb_w`` maps each head's latent output to ``v_head_dim``; the
    heads are concatenated (head-major) and multiplied by the o-projection
    rows of this rank's heads ("API Reference": ``out_absorb_w``, ``o_proj_w``)."""
    nh, dv, r = out_absorb_w.shape
    o_v = np.empty((nh, dv), dtype=F64)
    for h in range(nh):
        o_v[h] = out_absorb_w[h] @ o_lat[h]  # [dv, r] @ [r]
    return o_v.reshape(nh * dv) @ o_proj_w


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------

RowReader = Callable[[np.ndarray], np.ndarray]


def gather_keys(rows_t: np.ndarray, written: Dict[int, np.ndarray], read_rows: RowReader, kv_row: int) -> np.ndarray:
    """The cache rows one token attends over: one row per valid selected entry
    (duplicates kept, masked entries -1 skipped).  A row this step wrote reads
    the stored value, every other row the pool as it was before the step
    ("API Reference", ``kv_cache``: the cache is updated in place before the
    gather, so rows of this step are seen by it)."""
    valid = rows_t[rows_t >= 0]
    keys = np.empty((len(valid), kv_row))
    need = [i for i, rr in enumerate(valid.tolist()) if rr not in written]
    if need:
        keys[need] = read_rows(valid[need])
    for i, rr in enumerate(valid.tolist()):
        if rr in written:
            keys[i] = written[rr]
    return keys


def mla_gather_decode_step(inp: Dict[str, np.ndarray], read_rows: RowReader,
                           trace: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """One decode step for every token of the batch.

    ``inp`` maps the page's parameter names to float64 (values) / int64
    (indices) numpy arrays, plus the scalar parameters.  An optional
    ``token_seq`` [T] lets several tokens of one sequence share a step: token
    t resolves its selected positions through row ``token_seq[t]`` of
    ``block_table`` (then ``[n_seqs, max_blocks_per_seq]``); without it token
    t uses row t, one sequence per token as on the page ("Dimensions",
    ``n_tokens``).  ``read_rows(idx)``
    returns the pool's flat rows ``idx`` as float64 ``[len(idx), kv_row]``
    before this step; the rows the step writes are kept in an overlay, so the
    caller's pool is never modified.

    Order of effects: the front-fold of every token writes its row into the
    cache first, then the core gathers (the ``kv_cache`` parameter of "API
    Reference": the in-place update comes before the gather, so the gathered
    rows can include the ones stored in this step).  So a token that selects the position of another token of its
    sequence in this step (an earlier one; later ones are causally masked)
    reads that token's stored row, exactly as if the tokens had run as
    successive single-token steps in position order.

    Returns ``out [T, hidden]``, ``new_row [T, kv_row]`` (exact), ``stored_row``
    ``[T, kv_row]`` (bf16-rounded, as written), ``rows [T, n_prior]`` (flat row
    or -1 when masked) and ``mask [T, n_prior]`` (True where valid).
    """
    nh = int(inp["n_heads"])
    dn = int(inp["qk_nope_head_dim"])
    dr = int(inp["qk_rope_head_dim"])
    r = int(inp["kv_lora_rank"])
    scale = float(inp["softmax_scale"])
    eps = float(inp.get("norm_eps", 1e-6))
    x = inp["hidden_states"]
    T, H = x.shape
    bs = int(inp["kv_cache_block_size"])
    gi = inp["gather_indices"]
    P = gi.shape[1]
    kv_row = r + dr
    w = {k: inp[k] for k in ("input_norm_w", "wq_a", "q_norm_w", "wq_b", "wkv_a", "kv_norm_w",
                             "q_absorb_w", "out_absorb_w", "o_proj_w")}

    # front-fold for every token, then the cache-row writes
    q_lat = np.empty((T, nh, r))
    q_pe = np.empty((T, nh, dr))
    new_row = np.empty((T, kv_row))
    for t in range(T):
        q_lat[t], q_pe[t], _, new_row[t] = front_fold(
            x[t], w, inp["cos"][t], inp["sin"][t], nh, dn, dr, r, eps)
    stored = bf16_round(new_row)
    written = {}
    for t in range(T):
        written[int(inp["slot_mapping"][t])] = stored[t]

    # index build, gather, attention core, output projection
    seq = inp.get("token_seq")
    rows = np.full((T, P), -1, dtype=np.int64)
    out = np.empty((T, H))
    for t in range(T):
        pos = int(inp["positions"][t])
        table_row = inp["block_table"][t if seq is None else int(seq[t])]
        for j in range(P):
            rows[t, j] = resolve_row(int(gi[t, j]), pos, table_row, bs)
        keys = gather_keys(rows[t], written, read_rows, kv_row)
        o_lat = attention_core(q_lat[t], q_pe[t], keys, scale, r)
        out[t] = output_projection(o_lat, w["out_absorb_w"], w["o_proj_w"])
        if trace is not None:
            trace.setdefault("o_lat", []).append(o_lat)
    if trace is not None:
        trace["q_lat"] = q_lat
        trace["q_pe"] = q_pe
    return {"out": out, "new_row": new_row, "stored_row": stored, "rows": rows, "mask": rows >= 0}


# ---------------------------------------------------------------------------
# adapters for the torch tensors the workload generator produces
# ---------------------------------------------------------------------------

def to_f64_inputs(inp: Dict[str, object], block_size: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Widen a dict of torch tensors / scalars to the oracle's numpy form.

    The widening is exact (bf16 and fp32 are subsets of float64).  The cache
    pool is not converted; pass a row reader instead.
    """
    import torch

    out: Dict[str, np.ndarray] = {}
    if block_size is not None:
        out["kv_cache_block_size"] = int(block_size)
    for k, v in inp.items():
        if k == "kv_cache":
            out["kv_cache_block_size"] = int(v.shape[2])
            continue
        if isinstance(v, torch.Tensor):
            v = v.detach().cpu()
            if v.dtype in (torch.int32, torch.int64):
                out[k] = v.to(torch.int64).numpy()
            else:
                out[k] = v.to(torch.float64).numpy()
        else:
            out[k] = v
    for g in ("input_norm_w", "q_norm_w", "kv_norm_w"):
        if g in out:
            out[g] = out[g].reshape(-1)
    return out


def dense_row_reader(pool_rows_f64: np.ndarray) -> RowReader:
    """Row reader over a pool already widened to float64 ``[n_rows, kv_row]``."""
    return lambda idx: pool_rows_f64[np.asarray(idx, dtype=np.int64)]
