#!/usr/bin/env python3
"""Benchmark of one MLA gather-decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config all|NAME] [--fused] [--extras]
    python bench.py --traffic FETCH.csv WRITE.csv [--config NAME]   (offline, no GPU)

Prints ONE JSON line.  A "step" is one full pass of the path (index build,
front-fold, cache-row write, absorption, gather-attention core, output
absorption, o-projection) over one batch of synthetic, seeded inputs that are
resident in HBM before timing starts.  By default the line's ``value`` is the
DeepSeek-V3.2 slice (one token, 16 heads, n_prior 2048); ``configs`` holds the
same measurements for the other n_prior = 2048 workloads (32 tokens x 16
heads, 64 and 128 tokens x 128 heads), ``fused_ablation`` the single-launch
kv-row/absorption/core variant, ``single_launch_ablation`` the whole step as
one launch, ``router`` the fused RMSNorm + router top-K at one and 128 tokens,
``copy_GBps`` a plain device copy's bandwidth.

Timing: W warm-up steps, then K timed steps, every one of them preceded by a
read and write of a 1 GiB buffer so that neither the L2s nor the 256 MB
Infinity Cache hold the weights or the pool (cold-cache steps).  HIP events on
the step's stream bracket each step (the flush is outside them); ``value`` is
the median step latency in microseconds, kernels launched one by one
(``--graph``: the library replays its captured HIP graph).  K more
cold steps, each kernel launched with its own start and stop events (they
stamp the kernel's execution, not the dispatch gaps), give the per-kernel
breakdown.  Every dispatch of the run is a cold one, so a rocprofv3 kernel
trace of the same command averages the same launches.  ``--extras``
adds warm (back-to-back) and torch-captured graph timings.

``roofline`` is for the kernel with the largest mean duration: algorithmic
bytes per launch over its mean duration between its start and stop events,
against 8 TB/s.  ``core_mfma`` is the gather-attention core's algorithmic
flops (2 (kv_row + kv_lora_rank) n_heads per valid entry) over its mean
duration, against the 2.5 PFLOP/s dense bf16 peak.
``traffic`` is that kernel's HBM bytes per launch from two rocprofv3 counter
runs (FETCH_SIZE, WRITE_SIZE), scaled by what the same counters read for a
plain 512 MiB device copy, recorded by ``--traffic`` in profiles/traffic.json
with a digest of the kernel sources; it is null once the sources change.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA gather-decode step µs + achieved HBM GB/s (% of peak), n_prior=2048"
HBM_PEAK_GBPS = 8000.0


def alg_bytes(sh, inp, names) -> dict:
    """Algorithmic HBM bytes of one step, per kernel: every weight once, the
    gammas, activations in and out, the index tensors, the RoPE tables, each
    distinct valid gathered row once, and the written rows.  Split-K partials,
    query tiles and split-combine traffic are overheads and count nothing."""
    import numpy as np

    T, H, Q, r, dn, dr, dv, nh = (sh.n_tokens, sh.hidden, sh.q_lora_rank, sh.kv_lora_rank,
                                  sh.qk_nope_head_dim, sh.qk_rope_head_dim, sh.v_head_dim, sh.n_heads)
    kvr = r + dr
    P, MB = sh.n_prior, sh.max_blocks_per_seq
    gi = inp["gather_indices"].numpy()
    pos = inp["positions"].numpy()
    uniq = sum(len(np.unique(gi[t][(gi[t] >= 0) & (gi[t] <= pos[t])])) for t in range(T))
    inputs = 2 * T * H + 4 * H + 4 * T * P + 4 * T + 4 * T * MB  # x, g_in, gather_indices, positions, table
    kv_branch = 4 * Q + 4 * r + 4 * T * dr + 4 * T + 2 * T * kvr  # g_q, g_kv, cos+sin, slots, written rows
    w_down, w_qb = 2 * H * (Q + kvr), 2 * Q * nh * (dn + dr)
    if "k_prep" in names:  # matrix-core path
        b = {"k_prep": inputs, "k_down": w_down, "k_qa": kv_branch, "k_qup": w_qb}
    else:
        b = {"k_down": w_down + inputs, "k_qup": w_qb + kv_branch}
    b.update({"k_absorb": 2 * nh * dn * r, "k_core": 2 * kvr * uniq, "k_oabsorb": 2 * nh * dv * r,
              "k_oproj": 2 * nh * dv * H, "k_out": 2 * T * H})
    b["k_absorb_core"] = b["k_absorb"] + b["k_core"]  # the fused variant's single launch
    b["k_step"] = sum(b[n] for n in ("k_down", "k_qup", "k_absorb", "k_core", "k_oabsorb", "k_oproj", "k_out"))
    if "k_out" not in names:  # the GEMV path's o-projection writes the output itself
        b["k_oproj"] += b["k_out"]
    b = {n: b.get(n, 0) for n in names}
    b["step"] = sum(b.values())
    return b


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_gather_mla_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    w = rec.get(workload, {})
    # matrix-core-path kernels carry an _m in their symbol, the many-heads cores an _rs or _wide, the
    # one-token kernels compiled for the DeepSeek-V3.2 shape an _fx
    ent = (w.get(kernel) or w.get(kernel + "_m") or w.get(kernel + "_rs") or w.get(kernel + "_wide")
           or w.get(kernel + "_fx"))
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_launch")


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, inp_cpu, budget_s: float) -> dict:
    """The fp64 oracle, as it is, on the host cores, timed on a bounded sample
    of this workload's tokens (all of them up to 8 tokens, else the first 8),
    repeated until the budget is spent; once with the BLAS thread pool as
    configured and once on one thread.  The sampled tokens' cache rows are
    regenerated from the workload's counter-based pool in one untimed pass
    (the multi-GB pools are never materialised on the host); the timed passes
    gather them from that host table.  The weights are widened to fp64 once,
    outside the timed region.  ``value`` is microseconds per whole step: the
    time per token scaled by tokens per step (the oracle runs token by token)."""
    import numpy as np

    import oracle
    from workload import pool_rows

    sh = wl.shape
    T = sh.n_tokens
    o_all = oracle.to_f64_inputs({k: v for k, v in inp_cpu.items() if k != "kv_cache"},
                                 block_size=sh.block_size)
    per_token = ("hidden_states", "cos", "sin", "slot_mapping", "block_table", "positions", "gather_indices")
    toks = list(range(min(T, 8)))
    sample = {k: (v[toks] if k in per_token else v) for k, v in o_all.items()}
    table = {}

    def fetch(idx):  # untimed: regenerate and keep the rows the sample reads
        idx = np.asarray(idx, dtype=np.int64)
        vals = pool_rows(wl, idx).double().numpy()
        for i, r in enumerate(idx.tolist()):
            table[r] = vals[i]
        return vals

    oracle.mla_gather_decode_step(sample, fetch)

    def read(idx):
        return np.stack([table[r] for r in np.asarray(idx, dtype=np.int64).tolist()])

    def run(budget):
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.mla_gather_decode_step(sample, read)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return el / (reps * len(toks)) * T * 1e6, reps

    all_us, all_reps = run(budget_s)
    cores = _oracle_threads()
    one = None
    try:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1):
            one = run(max(1.0, budget_s / 2))
    except Exception:  # pragma: no cover
        pass
    what = (f"{len(toks)} of {T} tokens of {wl.name} (n_prior={sh.n_prior}), fp64 numpy, "
            f"gathering rows from a host table filled before timing; time per token x {T}")
    res = {"value": round(all_us, 1), "unit": "us", "cores": cores, "kind": "oracle",
           "sample": f"{all_reps} passes over {what}"}
    if one is not None:
        res["single_thread"] = {"value": round(one[0], 1), "unit": "us", "cores": 1,
                                "sample": f"{one[1]} passes, BLAS limited to one thread"}
    return res


COPY_CAL_BYTES = 512 << 20  # the calibration copy: reads and writes this many bytes


def traffic_from_counters(fetch_csv: str, write_csv: str, workload: str) -> int:
    """Offline: per-kernel HBM bytes per launch from two rocprofv3 counter CSVs
    (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) of a run with --calibrate-copy.
    Each counter is scaled so that the 512 MiB calibration copies read (write)
    exactly 512 MiB.  Writes profiles/traffic.json and prints a summary."""
    import csv

    def per_kernel(path, counter):
        vals, copies = {}, []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"])
                vals.setdefault(row["Kernel_Name"], []).append(v)
                if "copyBuffer" in row["Kernel_Name"]:
                    copies.append((int(row["Dispatch_Id"]), v))
        # the calibration copies are the run's last four copy-kernel dispatches
        cal = [v for _, v in sorted(copies)[-4:]]
        if len(cal) < 4 or min(cal) * 1024 < 0.2 * COPY_CAL_BYTES:
            raise SystemExit(f"{path}: no calibration copies at the end of the run")
        # the counter may read a fixed fraction of the bytes; that fraction is what the scale removes
        return vals, COPY_CAL_BYTES / (statistics.mean(cal) * 1024)

    fetch, sf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, sw = per_kernel(write_csv, "WRITE_SIZE")
    nf = nw = 4
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    ent = {}
    for k, v in fetch.items():
        short = k.split("(")[0].replace("void ", "").split("<")[0].strip()
        if not short.startswith("k_") or k not in write:
            continue
        f_kib, w_kib = statistics.mean(v), statistics.mean(write[k])
        ent[short] = {"bytes_per_launch": round(f_kib * 1024 * sf + w_kib * 1024 * sw),
                      "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
                      "dispatches": len(v), "source_digest": source_digest()}
    ent["_calibration"] = {"copy_bytes": COPY_CAL_BYTES, "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
                           "copies": [nf, nw]}
    rec[workload] = ent
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({workload: ent}, indent=1))
    return 0


def router_bench(args) -> int:
    """Cold latency of the fused RMSNorm + router top-K (two kernels), with the
    roofline of the whole call and the oracle timed on the host: one JSON line."""
    import json as _json

    print(_json.dumps(router_measure(args.router, args.steps, args.warmup, args.cpu_budget)), flush=True)
    return 0


def router_measure(name: str, steps: int, warmup: int, cpu_budget: float) -> dict:
    """The router line of ``router_bench`` as a dict (also nested in the default run's line)."""
    import statistics
    import time

    import numpy as np
    import torch

    from oracle import router_oracle as ro
    from sparse_gather_mla_amd.router import rmsnorm_router_topk, workspace_size
    from workload import ROUTER_CONFIGS, make_router_inputs

    T, H, E, K = ROUTER_CONFIGS[name]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = make_router_inputs(T, H, E, seed=31, with_bias=True)
    g = {k: v.to(dev) for k, v in inp.items()}
    out = (torch.empty((T, H), dtype=torch.bfloat16, device=dev), torch.empty((T, K), dtype=torch.int32, device=dev),
           torch.empty((T, E), dtype=torch.bfloat16, device=dev))
    ws = torch.zeros(workspace_size(T, H, E), dtype=torch.uint8, device=dev)
    flush = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev)

    def run():
        rmsnorm_router_topk(g["hidden_states"], g["gamma"], g["router_weights"], g["router_bias"], 1e-6, K,
                            "sigmoid", workspace=ws, out=out)

    for _ in range(warmup):
        flush.add_(1.0)
        run()
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        flush.add_(1.0)  # cold: evicts the L2s and the Infinity Cache
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    call_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    us = statistics.mean(call_us)
    # algorithmic bytes: weights, hidden states (read twice: GEMV and the normalised
    # write), gamma, bias, and the three outputs
    alg = 2 * H * E + 2 * 2 * T * H + 2 * H + 4 * E + 2 * T * H + 4 * T * K + 2 * T * E
    gemv_alg = 2 * H * E + 2 * T * H + 2 * H
    x = inp["hidden_states"].to(torch.float64).numpy()
    gam, w = inp["gamma"].to(torch.float64).numpy(), inp["router_weights"].to(torch.float64).numpy()
    bias = inp["router_bias"].to(torch.float64).numpy()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < min(cpu_budget, 10.0) or n == 0:
        ro.rmsnorm_router_topk(x, gam, w, bias, 1e-6, K, ro.SIGMOID)
        n += 1
    cpu_us = (time.perf_counter() - t0) / n * 1e6
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    q = np.percentile(call_us, [10, 50, 90])
    line = {"metric": "rmsnorm_router_topk_latency", "value": round(us, 3), "unit": "us", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": us / 1e3, "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "us_p10_p50_p90": [round(x, 3) for x in q],
            "config": {"workload": f"{name}: T={T}, H={H}, E={E}, top_k={K}, sigmoid, bias",
                       "cache_state": "cold (1 GiB flush per call)"},
            "roofline": {"bound": "hbm", "kernel": "whole call (k_rt_partial + k_rt_select)",
                         "achieved": round(alg / us / 1e3, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(alg / us / 1e3 / 8000.0, 4), "traffic": None, "alg_bytes": alg,
                         "gemv_alg_bytes": gemv_alg},
            "cpu_baseline": {"value": round(cpu_us, 1), "unit": "us", "cores": cores, "kind": "oracle",
                             "sample": f"{n} whole calls, fp64 numpy"}}
    del g, out, ws, flush
    torch.cuda.empty_cache()
    return line


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# the n_prior=2048 workloads of the metric: the headline one first
BENCH_CONFIGS = ("ds32_slice", "batch32", "fullhead64", "large128")


def core_flops(sh, inp) -> int:
    """Algorithmic flops of the gather-attention core: every valid entry
    (duplicates included, the softmax runs over the multiset) costs a score
    over the whole row and a value product over the latent, for every head."""
    import numpy as np

    gi = inp["gather_indices"].numpy()
    pos = inp["positions"].numpy()[:, None]
    valid = int(np.count_nonzero((gi >= 0) & (gi <= pos)))
    return 2 * valid * sh.n_heads * (sh.kv_row_dim + sh.kv_lora_rank)


def measure_config(name: str, steps: int, warmup: int, fused: bool = False, graph: bool = False,
                   extras: bool = False, cpu_budget: float = 0.0, calibrate_copy: bool = False,
                   single: bool = False, tokens: int = 0) -> dict:
    """Cold steps of one workload (its first ``tokens`` tokens if given): step
    latency (median, p10, p90, mean), the per-kernel breakdown from start/stop
    events on each kernel launch, the dominant kernel's roofline, the core's
    matrix-core utilisation and, with a budget, the oracle's host time.
    ``single``: the single-launch variant."""
    import numpy as np
    import torch

    from sparse_gather_mla_amd import Dims, MlaGatherDecode
    from workload import config_by_name, make_inputs, to_device

    wl = config_by_name(name)
    if tokens:
        wl = wl.with_tokens(tokens)
    sh = wl.shape
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, with_pool=False)  # the pool is filled on the GPU
    g = to_device(wl, inp, device=dev)
    mod = MlaGatherDecode(Dims.from_shape(sh), max_tokens=sh.n_tokens, device=0, fused=fused, graph=graph,
                          single_launch=single)
    names = mod.kernel_names(sh.n_tokens)
    nk = len(names)
    out = torch.empty((sh.n_tokens, sh.hidden), dtype=torch.bfloat16, device=dev)
    flush = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev)
    flush.zero_()
    stream = torch.cuda.current_stream(dev)

    # --- warm-up and timed steps, all cold ----------------------------------
    # The step as a caller runs it (kernels launched one by one; --graph: the
    # library replays its captured HIP graph), bracketed by events on its stream.
    W, K = warmup, steps
    bounds = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for _ in range(W):
        flush.add_(1.0)  # read + write 1 GiB: evicts the L2s and the Infinity Cache
        mod(g, out=out, stream=stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        flush.add_(1.0)
        bounds[k][0].record(stream)
        mod(g, out=out, stream=stream)
        bounds[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in bounds]

    # --- per-kernel breakdown: the same cold steps, each kernel launched with a
    # start and a stop event that stamp its own execution (no dispatch gaps);
    # these dispatches are the ones a kernel trace of this run averages too
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)] for _ in range(K)]
    for k in range(K):
        flush.add_(1.0)
        mod(g, out=out, events=evs[k], stream=stream)
    torch.cuda.synchronize()
    stage_ms = {names[i]: [evs[k][2 * i].elapsed_time(evs[k][2 * i + 1]) for k in range(K)] for i in range(nk)}
    direct_ms = [evs[k][0].elapsed_time(evs[k][2 * nk - 1]) for k in range(K)]

    res = {}
    if extras:
        # warm steps (no flush, back to back)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            mod(g, out=out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res["warm_us"] = round(e0.elapsed_time(e1) / K * 1e3, 3)
        # HIP graph of the step, cold
        try:
            gr = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                mod(g, out=out)  # warm the capture stream
                torch.cuda.synchronize()
                with torch.cuda.graph(gr, stream=side):
                    mod(g, out=out)
            torch.cuda.synchronize()
            gts = []
            for _ in range(K):
                flush.add_(1.0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                gr.replay()
                b.record(stream)
                gts.append((a, b))
            torch.cuda.synchronize()
            res["graph_cold_us"] = round(statistics.mean(a.elapsed_time(b) for a, b in gts) * 1e3, 3)
        except Exception as exc:  # pragma: no cover - reported, not fatal
            print(f"graph capture failed: {exc}", file=sys.stderr)

    if calibrate_copy:
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        src.fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(4):
            flush.add_(1.0)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ab = alg_bytes(sh, inp, names)
    q = np.percentile(step_ms, [10, 50, 90])
    med_ms = float(q[1])
    stage_us = {n: statistics.mean(v) * 1e3 for n, v in stage_ms.items()}
    dom = max(stage_us, key=stage_us.get)
    dom_bytes = ab.get(dom, 0)
    dom_gbps = dom_bytes / (stage_us[dom] * 1e-6) / 1e9
    step_gbps = ab["step"] / (med_ms * 1e-3) / 1e9
    res.update({
        "us": round(med_ms * 1e3, 3),
        "us_p10_p50_p90": [round(x * 1e3, 3) for x in q],
        "us_mean": round(statistics.mean(step_ms) * 1e3, 3),
        "workload": f"{wl.name}: {wl.description}",
        "n_tokens": sh.n_tokens, "n_heads": sh.n_heads,
        "achieved_GBps": round(step_gbps, 1),
        "pct_of_hbm_peak": round(100 * step_gbps / HBM_PEAK_GBPS, 2),
        "alg_bytes_per_step": ab["step"],
        "step_us_direct_launch_with_kernel_events": round(statistics.mean(direct_ms) * 1e3, 3),
        "wall_ms_per_step_incl_flush": round(wall / K * 1e3, 4),
        "stages": {n: {"us": round(stage_us[n], 3), "alg_bytes": ab.get(n, 0),
                       "GBps": round(ab.get(n, 0) / (stage_us[n] * 1e-6) / 1e9, 1)} for n in names},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom, wl.name), "alg_bytes_per_launch": dom_bytes},
    })
    core = next((n for n in names if n.startswith("k_core") or n == "k_absorb_core"), None)
    if core is not None:
        fl = core_flops(sh, inp)
        tf = fl / (stage_us[core] * 1e-6) / 1e12
        res["core_mfma"] = {"kernel": core, "alg_flops": fl, "us": round(stage_us[core], 3),
                            "achieved_TFLOPs": round(tf, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "utilisation": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    del g, mod, flush
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(wl, inp, cpu_budget)
    return res


def copy_bandwidth_gbps(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Attainable HBM bandwidth of a plain device-to-device copy (read + write)."""
    import torch

    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="all",
                    help="one workload, or 'all': ds32_slice as the headline plus the other n_prior=2048 configs")
    ap.add_argument("--fused", action="store_true")
    ap.add_argument("--single", action="store_true", help="the single-launch variant (whole step, one kernel)")
    ap.add_argument("--graph", action="store_true", help="the library captures the step once and replays it")
    ap.add_argument("--extras", action="store_true", help="also time warm steps and a HIP graph of the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with four plain 512 MiB device copies (for counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--router", default=None, metavar="NAME",
                    help="time the fused RMSNorm + router top-K instead (router_t1 or router_t128)")
    args = ap.parse_args()

    if args.traffic:
        return traffic_from_counters(args.traffic[0], args.traffic[1],
                                     "ds32_slice" if args.config == "all" else args.config)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the step is single-GPU; the multi-GPU design is documented, not built)", file=sys.stderr)
        return 2

    if args.router:
        return router_bench(args)

    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    head_name = "ds32_slice" if args.config == "all" else args.config
    print(f"[bench] {head_name}: {args.warmup} + {args.steps} cold steps", file=sys.stderr, flush=True)
    head = measure_config(head_name, args.steps, args.warmup, fused=args.fused, graph=args.graph,
                          extras=args.extras, cpu_budget=budget,
                          calibrate_copy=args.calibrate_copy and args.config != "all", single=args.single)
    res = {
        "metric": METRIC,
        "value": head["us"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "n_tokens": head["n_tokens"], "n_heads": head["n_heads"],
                   "n_prior": 2048,
                   "variant": "fused" if args.fused else ("single launch" if args.single else "separate"),
                   "cache_state": "cold (1 GiB flush per step)",
                   "statistic": "median of the timed steps"},
        "launch": "captured HIP graph, replayed" if args.graph else "kernels launched one by one",
    }
    for k in ("us_p10_p50_p90", "us_mean", "achieved_GBps", "pct_of_hbm_peak", "alg_bytes_per_step",
              "step_us_direct_launch_with_kernel_events", "wall_ms_per_step_incl_flush", "stages", "roofline",
              "core_mfma", "warm_us", "graph_cold_us"):
        if k in head:
            res[k] = head[k]
    res["accumulate"] = "fp32"
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
    if args.config == "all":
        copy_gbps = copy_bandwidth_gbps()
        res["copy_GBps"] = round(copy_gbps, 1)
        res["pct_of_copy_bandwidth"] = round(100 * head["achieved_GBps"] / copy_gbps, 2)
        if not args.fused and not args.single:
            # the ablation of the pages: kv-row write, absorption and core fused in one launch
            print("[bench] ds32_slice fused variant", file=sys.stderr, flush=True)
            fz = measure_config(head_name, args.steps, args.warmup, fused=True)
            res["fused_ablation"] = {"separate_us": head["us"], "fused_us": fz["us"],
                                     "fused_us_p10_p50_p90": fz["us_p10_p50_p90"],
                                     "fused_stages": {n: v["us"] for n, v in fz["stages"].items()},
                                     "pages_context_us": {"separate": 385.8, "fused": 340.2,
                                                          "hardware": "AWS Neuron, unstated shape"}}
            # the whole step as one launch, against the separate kernels: ds32_slice
            # and the batch32 workload cut to 3 tokens (the most the variant takes)
            sl = {}
            for name, tok, sep_us in ((head_name, 0, head["us"]), ("batch32", 3, None)):
                label = name if not tok else f"{name}_T{tok}"
                if sep_us is None:
                    print(f"[bench] {label} separate kernels", file=sys.stderr, flush=True)
                    sep_us = measure_config(name, args.steps, args.warmup, tokens=tok)["us"]
                print(f"[bench] {label} single launch", file=sys.stderr, flush=True)
                one = measure_config(name, args.steps, args.warmup, single=True, tokens=tok)
                sl[label] = {"separate_us": sep_us, "single_launch_us": one["us"],
                             "single_launch_us_p10_p50_p90": one["us_p10_p50_p90"]}
            res["single_launch_ablation"] = sl
        res["configs"] = {}
        for name in BENCH_CONFIGS[1:]:
            # the 128-head workloads keep the run short: fewer steps
            k = args.steps if name == "batch32" else max(5, args.steps // 2)
            print(f"[bench] {name}: {args.warmup} + {k} cold steps", file=sys.stderr, flush=True)
            c = measure_config(name, k, args.warmup, cpu_budget=budget / 2)
            c["pct_of_copy_bandwidth"] = round(100 * c["achieved_GBps"] / copy_gbps, 2)
            res["configs"][name] = c
        # the widening beside the step: the fused RMSNorm + MoE router top-K (mean of cold calls)
        res["router"] = {}
        for name in ("router_t1", "router_t128"):
            print(f"[bench] {name}: {args.warmup} + {args.steps} cold calls", file=sys.stderr, flush=True)
            r = router_measure(name, args.steps, args.warmup, min(budget, 2.0))
            res["router"][name] = {k: r[k] for k in ("value", "unit", "us_p10_p50_p90", "config", "roofline",
                                                     "cpu_baseline")}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
