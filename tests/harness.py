"""Helpers shared by the GPU parity tests, the smoke check and the benchmark's
CPU-baseline leg: draw a workload, run the fp64 oracle on chosen tokens, run
the HIP library, and compare the two.
"""
from __future__ import annotations

import time
from typing import Dict, Iterable, List, Optional

import numpy as np
import torch

import oracle
from workload import Workload, fill_pool_, make_inputs, pool_rows

# Acceptance bar: max |err| <= TOL * RMS(reference) on the bf16 output and on the
# bf16 cache-row values (fp32 accumulation on the GPU).
TOL = 2e-2


def rms(a: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def within_tol(got: np.ndarray, ref: np.ndarray, tol: float = TOL):
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0
    bound = tol * rms(ref)
    return err <= bound and np.all(np.isfinite(got)), err, bound


def token_slice(inp: Dict[str, object], tokens: Iterable[int]) -> Dict[str, object]:
    """Inputs restricted to some tokens (tokens are independent sequences)."""
    idx = torch.as_tensor(list(tokens), dtype=torch.long)
    per_token = ("hidden_states", "cos", "sin", "slot_mapping", "block_table", "positions", "gather_indices")
    out = {}
    for k, v in inp.items():
        if k == "kv_cache":
            continue
        out[k] = v[idx.to(v.device)] if k in per_token else v
    return out


def oracle_reference(wl: Workload, inp_cpu: Dict[str, object], tokens: List[int],
                     pool_cpu: Optional[torch.Tensor] = None) -> Dict[str, np.ndarray]:
    """Run the oracle on the given tokens.  Rows come from `pool_cpu` if given,
    else they are regenerated from the workload's counter-based pool."""
    sub = token_slice(inp_cpu, tokens)
    o = oracle.to_f64_inputs(sub, block_size=wl.shape.block_size)
    kvr = wl.shape.kv_row_dim
    if pool_cpu is not None:
        flat = pool_cpu.view(-1, kvr)

        def reader(idx):
            return flat[torch.from_numpy(np.asarray(idx, dtype=np.int64))].double().numpy()
    else:
        def reader(idx):
            return pool_rows(wl, np.asarray(idx)).double().numpy()
    return oracle.mla_gather_decode_step(o, reader)


def gpu_inputs(wl: Workload, inp_cpu: Dict[str, object], device="cuda") -> Dict[str, object]:
    """Copy the small tensors to the GPU and fill the pool there."""
    sh = wl.shape
    g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp_cpu.items() if k != "kv_cache"}
    if "kv_cache" in inp_cpu:
        g["kv_cache"] = inp_cpu["kv_cache"].to(device)
    else:
        pool = torch.empty((sh.n_blocks, 1, sh.block_size, sh.kv_row_dim), dtype=torch.bfloat16, device=device)
        g["kv_cache"] = fill_pool_(wl, pool)
    return g


def index_build_all(inp_cpu: Dict[str, object], block_size: int) -> np.ndarray:
    """Every token's flat rows via the oracle's per-entry index build."""
    gi = inp_cpu["gather_indices"].numpy()
    pos = inp_cpu["positions"].numpy()
    bt = inp_cpu["block_table"].numpy()
    T, P = gi.shape
    rows = np.empty((T, P), dtype=np.int64)
    for t in range(T):
        p = int(pos[t])
        for j in range(P):
            rows[t, j] = oracle.resolve_row(int(gi[t, j]), p, bt[t], block_size)
    return rows


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0
