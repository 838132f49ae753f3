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
from workload import Workload, make_inputs, pool_rows, to_device

# Acceptance bar: max |err| <= TOL * RMS(reference) on the bf16 output and on the
# bf16 cache-row values (fp32 accumulation on the GPU).
TOL = 2e-2


def rms(a: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at each value: the distance below which no bf16
    number can come to it (|x| in [2^(E-1), 2^E) has spacing 2^(E-8))."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, e - 9)


def within_tol(got: np.ndarray, ref: np.ndarray, tol: float = TOL):
    """The acceptance bar on a bf16 result against the fp64 reference: per
    element, |got - ref| <= tol * RMS(ref) + half a bf16 spacing at ref.  The
    second term is the format's own floor: even the correctly rounded
    reference misses ref by up to half a spacing, which exceeds tol * RMS for
    elements beyond about 5 RMS (|ref| >= 2^k with 2^(k-8) > tol * RMS).
    Returns (ok, max |got - ref|, tol * RMS(ref))."""
    got = got.astype(np.float64)
    if not got.size:
        return True, 0.0, 0.0
    d = np.abs(got - ref)
    bound = tol * rms(ref)
    ok = bool(np.all(d <= bound + bf16_half_ulp(ref))) and bool(np.all(np.isfinite(got)))
    return ok, float(np.max(d)), bound


def token_slice(inp: Dict[str, object], tokens: Iterable[int]) -> Dict[str, object]:
    """Inputs restricted to some tokens.  With token_seq the block table is
    per sequence and stays whole (the kept tokens index into it)."""
    idx = torch.as_tensor(list(tokens), dtype=torch.long)
    per_token = ("hidden_states", "cos", "sin", "slot_mapping", "positions", "gather_indices", "token_seq")
    if "token_seq" not in inp:
        per_token = per_token + ("block_table",)
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
    return to_device(wl, inp_cpu, device)


def index_build_all(inp_cpu: Dict[str, object], block_size: int) -> np.ndarray:
    """Every token's flat rows via the oracle's per-entry index build."""
    gi = inp_cpu["gather_indices"].numpy()
    pos = inp_cpu["positions"].numpy()
    bt = inp_cpu["block_table"].numpy()
    T, P = gi.shape
    seq = inp_cpu["token_seq"].numpy() if inp_cpu.get("token_seq") is not None else np.arange(T)
    rows = np.empty((T, P), dtype=np.int64)
    for t in range(T):
        p = int(pos[t])
        for j in range(P):
            rows[t, j] = oracle.resolve_row(int(gi[t, j]), p, bt[int(seq[t])], block_size)
    return rows


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0
