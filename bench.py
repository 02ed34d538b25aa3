#!/usr/bin/env python3
"""Benchmark of the fused IPA forward on one MI355X.

One step = one full forward over one batch: ipa_lift (frames -> lifted
operands) followed by ipa_attend (fused online-softmax attention + output
epilogue), on inputs already resident in device memory.

Prints ONE JSON line: throughput in residue pairs per second (all heads, the
whole job) on the 2048-residue chain, achieved TFLOP/s against the
algorithmic count 2 H (d_qk + d_v) sum_b n_b^2 with d_qk = C + 3 Pqk + 2 +
R Cz and d_v = C + 3 Pv + R Cz, the roofline of the dominant kernel
(ipa_attend) from HIP events recorded on its own stream, the same figures for
the other workload sizes (512, 4096, the ragged batch, 8192 and 16384
residues), the other entry points (distance attention, frames, layer,
gradient, direction-and-distance attention), peak device memory versus L,
and the fp64 CPU oracle timed on the host's cores as a reported baseline.

Order of work: the CPU oracle runs first, before anything touches the GPU
(its worker processes are forked from a process without a GPU context); then
every GPU measurement runs back to back, the headline last, so that its
timed steps see the clocks the chip holds under sustained load rather than
the ramp of a cold start.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# MI355X fp32 vector peak without packed fp32 instructions (this library is
# built without them): 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2.4 GHz.
PEAK_FP32_VECTOR_TFLOPS = 78.6
PEAK_FP32_MFMA_TFLOPS = 157.3    # MI355X dense fp32 matrix peak
METRIC = "IPA fwd pairs/s & TFLOP/s (% bf16 MFMA peak) at L=2048; peak HBM GB vs L"
HEADLINE = "long_chain_2048"
# the other workload sizes, timed like the headline and reported beside it
# (the longest last: the headline follows it directly)
CONFIGS = ("single_chain", "ragged_batch", "long_chain_4096", "very_long_8192", "very_long_16384")


def algo_flops(d: dict, pairs: int) -> float:
    dqk = d["C"] + 3 * d["Pqk"] + 2 + d["R"] * d["Cz"]
    dv = d["C"] + 3 * d["Pv"] + d["R"] * d["Cz"]
    return 2.0 * d["H"] * (dqk + dv) * pairs


def algo_bytes(d: dict, elem: int = 2) -> float:
    """Algorithmic HBM bytes of one forward: read every input once, write
    every output once (inputs in storage precision, frames/outputs fp32)."""
    B, L, H, C, Pqk, Pv, R, Cz = (d[k] for k in ("B", "L", "H", "C", "Pqk", "Pv", "R", "Cz"))
    per_res_in = elem * (3 * H * C + H * 3 * (2 * Pqk + Pv) + 2 * R * Cz) + 4 * 12 + 1
    per_res_out = 4 * H * (C + 3 * Pv + Pv + Cz)
    return float(B * L * (per_res_in + per_res_out) + 4 * (Cz * H + H))


# Hardware byte counters of the dominant kernel, taken with rocprofv3 (one
# FETCH_SIZE pass, one WRITE_SIZE pass) per workload and committed as a
# summary together with the hash of the kernel source they were taken on
# (the attention kernel, its launcher and the workspace layout it reads: the
# whole of ipa_attn.hip and ipa_internal.h up to the gradient's argument
# block, which the attention does not include).
KERNEL_SOURCES = ("ipa_attn.hip", "ipa_internal.h")
_INTERNAL_CUT = b"struct BwdArgs"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "geometric_invariant_attention_amd", "csrc", f), "rb") as fh:
            data = fh.read()
        if f == "ipa_internal.h" and _INTERNAL_CUT in data:
            data = data[:data.index(_INTERNAL_CUT)]
        h.update(data)
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes of one ipa_attend launch from the committed counter summary
    of this workload (each counter scaled by what it reads for a plain copy
    of known size), or None when there is none or it was taken on kernel
    source that has changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", f"ipa_attend_{workload}_pmc.md")) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
            if rec.get("workload") != workload or rec.get("kernel_source_sha256") != kernel_source_hash():
                return None
            read_b = rec["fetch_kib_per_launch"] * 1024 * rec["fetch_scale"]
            write_b = rec["write_kib_per_launch"] * 1024 * rec["write_scale"]
            return {"bytes": read_b + write_b, "read_bytes": read_b, "write_bytes": write_b}
    return None


# ---------------------------------------------------------------------------
# CPU side: the fp64 oracle, timed before the GPU is touched
# ---------------------------------------------------------------------------

def cpu_workers() -> int:
    """Worker processes for the oracle: the cores this process may run on,
    at most 16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# inputs by workload name, filled before the pool forks so that every worker
# inherits them
_CPU_INPUTS: dict = {}


def _worker_init():
    from threadpoolctl import threadpool_limits
    global _WORKER_LIMITS
    _WORKER_LIMITS = threadpool_limits(limits=1)


def _oracle_rows(name: str, rows):
    from oracle import ipa_forward as oracle_forward
    t0 = time.perf_counter()
    ref = oracle_forward(_CPU_INPUTS[name], rows=rows)
    return rows, ref, time.perf_counter() - t0


def cpu_headline(pool, P: int, name: str, budget_s: float) -> dict:
    """The oracle on a bounded sample of the headline workload's query rows
    (every row is independent), spread over P single-threaded workers."""
    import numpy as np
    inp = _CPU_INPUTS[name]
    L, B = inp["dims"]["L"], inp["dims"]["B"]
    order = np.random.default_rng(1234).permutation(L)
    done, n, rows_all, refs = 0, 4, [], []
    t0 = time.perf_counter()
    while done < L and time.perf_counter() - t0 < budget_s:
        chunks = [np.sort(order[done + k * n: done + (k + 1) * n]) for k in range(P)]
        chunks = [c for c in chunks if len(c)]
        for rows, ref, _ in pool.starmap(_oracle_rows, [(name, c) for c in chunks]):
            rows_all.append(rows)
            refs.append(ref)
            done += len(rows)
        n = min(2 * n, 32)
    wall = time.perf_counter() - t0
    pairs = B * done * L
    return {
        "baseline": {
            "value": pairs / wall, "unit": "pairs/s", "cores": P, "kind": "oracle",
            "threads": {"workers": P, "blas_threads_per_worker": 1}, "cpu_model": cpu_model(),
            "sample": f"{done} of {L} query rows x {L} keys x B={B} (all {inp['dims']['H']} heads) of {name}, "
                      f"fp64 numpy oracle split by query rows over {P} processes, {wall:.1f} s wall",
        },
        "rows": rows_all, "refs": refs,
    }


def cpu_single_thread(name: str, budget_s: float) -> dict:
    """The oracle on one core (one process, one BLAS thread) on query rows of
    the 512-residue chain."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import ipa_forward as oracle_forward
    inp = _CPU_INPUTS[name]
    L, B = inp["dims"]["L"], inp["dims"]["B"]
    order = np.random.default_rng(99).permutation(L)
    done, n, spent = 0, 8, 0.0
    with threadpool_limits(limits=1):
        while done < L and spent < budget_s:
            rows = np.sort(order[done:done + n])
            t0 = time.perf_counter()
            oracle_forward(inp, rows=rows)
            spent += time.perf_counter() - t0
            done += len(rows)
            n = min(2 * n, 128)
    return {"value": B * done * L / spent, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "threads": {"workers": 1, "blas_threads_per_worker": 1}, "cpu_model": cpu_model(),
            "sample": f"{done} of {L} query rows x {L} keys of {name} (all heads), one core, {spent:.1f} s"}


def config_sample_rows(inp, n: int = 512):
    """Query rows on which the oracle times and checks a workload size: all
    of them up to 2048 residues, otherwise a seeded sample of n rows that
    includes the tile and block edges of the first and last four 64-residue
    blocks."""
    import numpy as np
    L = inp["dims"]["L"]
    if L <= 2048:
        return np.arange(L, dtype=np.int64)
    edges = set()
    for t in list(range(0, 4 * 64, 64)) + list(range(L - 4 * 64, L, 64)):
        edges.update({t, t + 1, t + 31, t + 32, t + 63})
    edges = {r for r in edges if 0 <= r < L}
    rng = np.random.default_rng(77)
    rest = rng.choice(np.setdiff1d(np.arange(L), np.array(sorted(edges))), size=n - len(edges), replace=False)
    return np.array(sorted(edges | set(int(x) for x in rest)), dtype=np.int64)


def cpu_config(pool, P: int, name: str) -> dict:
    """The oracle on the rows config_sample_rows picks for a workload size,
    split over P single-threaded workers: its timing (per pair, scaled from
    the sample when it is one) and its outputs for the GPU's parity."""
    import numpy as np
    inp = _CPU_INPUTS[name]
    L, B = inp["dims"]["L"], inp["dims"]["B"]
    rows = config_sample_rows(inp)
    chunks = [c for c in np.array_split(rows, P) if len(c)]
    t0 = time.perf_counter()
    parts = pool.starmap(_oracle_rows, [(name, c) for c in chunks])
    wall = time.perf_counter() - t0
    ref = {k: np.concatenate([pr[1][k] for pr in parts], axis=1) for k in parts[0][1]}
    full = len(rows) == L
    return {
        "baseline": {
            "value": B * len(rows) * L / wall, "unit": "pairs/s", "cores": P, "kind": "oracle",
            "threads": {"workers": P, "blas_threads_per_worker": 1},
            "sample": (f"the whole workload ({B} x {L} x {L} pairs)" if full else
                       f"{len(rows)} of {L} query rows x {L} keys x B={B}, extrapolated per pair")
                      + f", {wall:.2f} s wall",
        },
        "rows": rows, "ref": ref,
    }


def _threads_note(P: int) -> dict:
    return {"workers": 1, "blas_threads": P, "torch_threads": P}


def cpu_meet(P: int) -> dict:
    import numpy as np
    from oracle import meet_attention
    from workloads import MEET_WORKLOADS, make_meet_inputs
    w = MEET_WORKLOADS["meet_chain_2048"]
    inp = make_meet_inputs(w)
    d = w.dims()
    t0 = time.perf_counter()
    ref = meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"])
    wall = time.perf_counter() - t0
    pairs = d["B"] * d["L"] * d["L"]
    return {"baseline": {"value": pairs / wall, "unit": "pairs/s", "cores": P, "kind": "oracle",
                         "threads": _threads_note(P),
                         "sample": f"the whole {w.name} workload ({d['L']} x {d['L']} pairs, {d['H']} heads), "
                                   f"{wall:.2f} s"},
            "ref": np.asarray(ref)}


def cpu_frames(P: int) -> dict:
    from oracle import frames_from_atoms
    from workloads import make_backbone
    B, L = 16, 16384
    bb = make_backbone(B, L, seed=0)
    t0 = time.perf_counter()
    r_ref, _ = frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    wall = time.perf_counter() - t0
    return {"baseline": {"value": B * L / wall, "unit": "residues/s", "cores": P, "kind": "oracle",
                         "threads": _threads_note(P),
                         "sample": f"the whole workload ({B * L} residues), {wall:.2f} s"},
            "ref": r_ref}


def cpu_layer(P: int) -> dict:
    from oracle import ipa_layer
    from workloads import WORKLOADS, make_layer_inputs
    ci = make_layer_inputs(WORKLOADS[HEADLINE].with_(L=256), c_s=384)
    t0 = time.perf_counter()
    ipa_layer(ci)
    wall = time.perf_counter() - t0
    return {"baseline": {"value": 256 * 256 / wall, "unit": "pairs/s", "cores": P, "kind": "oracle",
                         "threads": _threads_note(P),
                         "sample": f"fp64 layer oracle on a 256-residue chain with the headline's dimensions "
                                   f"(c_s = 384), {wall:.2f} s, scaled per pair"}}


def cpu_backward(P: int) -> dict:
    import numpy as np
    from oracle import ipa_backward as oracle_backward
    from workloads import WORKLOADS, make_inputs
    ws = WORKLOADS[HEADLINE].with_(L=256)
    ci = make_inputs(ws)
    d = ws.dims()
    shapes = {"s": (d["C"],), "pts": (d["Pv"], 3), "pts_norm": (d["Pv"],), "pair": (d["Cz"],)}
    rng = np.random.default_rng(1)
    cg = {k: rng.standard_normal((ws.B, ws.L, d["H"]) + v) for k, v in shapes.items()}
    t0 = time.perf_counter()
    oracle_backward(ci, cg)
    wall = time.perf_counter() - t0
    return {"baseline": {"value": ws.B * ws.L * ws.L / wall, "unit": "pairs/s", "cores": P, "kind": "oracle",
                         "threads": _threads_note(P),
                         "sample": f"fp64 autograd oracle on a {ws.L}-residue chain with the same H, C, points "
                                   f"and pair factors, {wall:.1f} s, scaled per pair"}}


DD_NAMES = ("rot", "trans", "q_direction", "k_direction", "q_point", "k_point", "values",
            "direction_scale", "distance_scale", "output_weight", "output_bias")


def cpu_dirdist(P: int, budget_s: float = 8.0) -> dict:
    import numpy as np
    from oracle import dirdist_attention
    from workloads import DIRDIST_WORKLOADS, make_dirdist_inputs
    w = DIRDIST_WORKLOADS["dd_chain_2048"]
    inp = make_dirdist_inputs(w)
    d = w.dims()
    order = np.random.default_rng(7).permutation(d["N"])
    done, spent, n, rows_all, refs = 0, 0.0, 16, [], []
    while done < d["N"] and spent < budget_s:
        rows = np.sort(order[done:done + n])
        t0 = time.perf_counter()
        ref = dirdist_attention(**{k: inp[k] for k in DD_NAMES}, frame_mask=inp["frame_mask"], rows=rows)
        spent += time.perf_counter() - t0
        rows_all.append(rows)
        refs.append(ref)
        done += len(rows)
        n = min(2 * n, 256)
    return {"baseline": {"value": d["B"] * done * d["N"] / spent, "unit": "pairs/s", "cores": P,
                         "kind": "oracle", "threads": _threads_note(P),
                         "sample": f"{done} of {d['N']} query rows x {d['N']} keys, all {d['H']} heads, "
                                   f"fp64 numpy, {spent:.1f} s"},
            "rows": rows_all, "refs": refs}


def run_cpu_side(args, P: int) -> dict:
    """Every oracle timing and every oracle output that a GPU result is
    later compared with, computed before the GPU is initialised."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    from workloads import WORKLOADS, make_inputs

    res = {"P": P}
    names = [args.workload] + ([] if args.only_headline else [c for c in CONFIGS if c != args.workload])
    for nm in names:
        _CPU_INPUTS[nm] = make_inputs(WORKLOADS[nm])
    ctx = mp.get_context("fork")
    with ctx.Pool(P, initializer=_worker_init) as pool:
        res["headline"] = cpu_headline(pool, P, args.workload, args.cpu_budget)
        print(f"[bench] cpu oracle {res['headline']['baseline']['value']:.3e} pairs/s on {P} cores "
              f"({res['headline']['baseline']['sample']})", file=sys.stderr, flush=True)
        # the other sizes: the oracle's timing and the rows their GPU
        # outputs are checked on
        res["configs"] = {nm: cpu_config(pool, P, nm) for nm in names[1:]}
    if args.only_headline:
        return res
    if "single_chain" not in _CPU_INPUTS:
        _CPU_INPUTS["single_chain"] = make_inputs(WORKLOADS["single_chain"])
    res["single_thread"] = cpu_single_thread("single_chain", min(10.0, args.cpu_budget))
    print(f"[bench] cpu oracle, one core: {res['single_thread']['value']:.3e} pairs/s", file=sys.stderr,
          flush=True)
    import torch
    nt = torch.get_num_threads()
    torch.set_num_threads(P)
    with threadpool_limits(limits=P):
        res["meet"] = cpu_meet(P)
        res["frames"] = cpu_frames(P)
        res["layer"] = cpu_layer(P)
        res["backward"] = cpu_backward(P)
        res["dirdist"] = cpu_dirdist(P)
    torch.set_num_threads(nt)
    print("[bench] cpu side done", file=sys.stderr, flush=True)
    del np
    return res


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

def to_device(inp, dev):
    import numpy as np
    import torch
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dt).to(dev)
         for k in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2")}
    for k in ("rot", "trans", "w_b", "gamma"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
    t["mask"] = torch.from_numpy(inp["mask"]).to(dev) if inp.get("has_mask") else None
    return t


def prepare(w, dev, inp=None):
    """Inputs of workload w on the device and a bound forward plan."""
    import torch
    from geometric_invariant_attention_amd import IPAForward
    from workloads import make_inputs

    if inp is None:
        inp = make_inputs(w)
    t = to_device(inp, dev)
    d = w.dims()
    plan = IPAForward(**d, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = plan.bind(**{k: t[k] for k in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans",
                                          "z1", "z2", "w_b", "gamma")},
                    mask=t["mask"], w_L=inp["w_L"], w_C=inp["w_C"], stream=stream)
    return {"w": w, "inp": inp, "t": t, "plan": plan, "raw": raw, "stream": stream}


def time_steps(prep, steps: int, warmup: int, dev):
    """`warmup` untimed forwards, then exactly `steps` timed ones; then the
    per-kernel durations. The outputs stay on the device (plan.out)."""
    import torch
    plan, raw, stream = prep["plan"], prep["raw"], prep["stream"]
    for _ in range(warmup):
        plan.lift_raw(raw)
        plan.attend_raw(raw)
    torch.cuda.synchronize(dev)
    # timed region: exactly `steps` forwards, nothing else enqueued between
    # the kernels (an event record between two dependent kernels costs a few
    # microseconds of its own)
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.lift_raw(raw)
        plan.attend_raw(raw)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    # per-kernel durations: each kernel launched `steps` times back to back
    # between two HIP events on its own stream (both kernels only read what
    # the lift wrote from the inputs, so repeating either is the same work);
    # an event record between two dependent kernels would add the dispatch
    # latency of the second to its measured duration
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    for _ in range(steps):
        plan.lift_raw(raw)
    ev[1].record(stream)
    ev[2].record(stream)
    for _ in range(steps):
        plan.attend_raw(raw)
    ev[3].record(stream)
    torch.cuda.synchronize(dev)
    return wall, ev[0].elapsed_time(ev[1]) / steps, ev[2].elapsed_time(ev[3]) / steps


def outputs(prep) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in prep["plan"].out.items()}


def parity_on_rows(out, rows_list, refs) -> dict:
    import numpy as np
    errs = {}
    for rows, ref in zip(rows_list, refs):
        for k in ref:
            e = float(np.abs(out[k][:, rows].astype(np.float64) - ref[k]).max())
            errs[k] = max(errs.get(k, 0.0), e)
    return errs


def step_figures(w, inp, wall, steps, lift_ms, attn_ms) -> dict:
    """Per-step throughput and the attention kernel's roofline figures."""
    d = w.dims()
    pairs = int((inp["lengths"].astype("int64") ** 2).sum())
    flops = algo_flops(d, pairs)
    ms_step = wall * 1e3 / steps
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    nbytes = algo_bytes(d, 2 if w.dtype == "bf16" else 4)
    traffic = measured_traffic(w.name)
    fig = {
        "ms_per_step": ms_step, "pairs": pairs, "pairs_per_s": pairs / (ms_step * 1e-3),
        "head_pairs_per_s": d["H"] * pairs / (ms_step * 1e-3),
        "tflops": flops / (ms_step * 1e-3) / 1e12, "pct_bf16_peak": 100.0 * flops / (ms_step * 1e-3) / 1e12
        / PEAK_MFMA_TFLOPS,
        "kernels_ms": {"ipa_lift": lift_ms, "ipa_attend": attn_ms},
        "attend_roofline": {"kernel": "ipa_attend", "bound": "mfma", "achieved": attn_tflops,
                            "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": attn_tflops / PEAK_MFMA_TFLOPS,
                            "traffic": traffic["bytes"] if traffic else None, "algorithmic_flops": flops},
        "step_hbm": {"algorithmic_bytes": nbytes, "achieved_GBs": nbytes / (ms_step * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "frac": nbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }
    if traffic:
        fig["attend_hbm_GBs_counters"] = traffic["bytes"] / (attn_ms * 1e-3) / 1e9
    return fig


def bench_config(name: str, dev, steps: int, warmup: int):
    """Time one workload size; returns its figures and its prepared plan
    (outputs still on the device, checked later by config_parity)."""
    from workloads import WORKLOADS
    w = WORKLOADS[name]
    prep = prepare(w, dev, inp=_CPU_INPUTS.get(name))
    wall, lift_ms, attn_ms = time_steps(prep, steps, warmup, dev)
    res = {"workload": name, "config": {**w.dims(), "storage": w.dtype,
                                        "ragged": list(w.ragged) if w.ragged else None},
           **step_figures(w, prep["inp"], wall, steps, lift_ms, attn_ms)}
    if name == "ragged_batch":
        # short rows: the step is bound by memory traffic and latency, not
        # by the products
        h = res["step_hbm"]
        res["roofline"] = {"bound": "hbm", "achieved": h["achieved_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": h["frac"], "algorithmic_bytes": h["algorithmic_bytes"],
                           "note": "whole step (lift + attend), algorithmic bytes: every input read once, "
                                   "every output written once"}
    print(f"[bench] {name}: {res['ms_per_step'] * 1e3:.1f} us/step, attend "
          f"{res['attend_roofline']['frac']:.3f} of bf16 peak", file=sys.stderr, flush=True)
    return res, prep


def config_parity(res: dict, prep, cpu) -> None:
    if cpu is None:
        return
    rows, ref = cpu["rows"], cpu["ref"]
    # rows whose own mask entry is 0 are compared too (both sides give +0.0)
    res["cpu_baseline"] = cpu["baseline"]
    res["parity_on_rows"] = {"rows": len(rows), "max_abs_err": parity_on_rows(outputs(prep), [rows], [ref]),
                             "tol": 3e-2 if prep["w"].dtype == "bf16" else 1e-4}


def bench_meet(dev, steps: int, warmup: int, cpu) -> dict:
    """Distance-penalised attention (ipa_meet_forward) on the 2048-residue
    chain: the forward timed like the IPA step, the fp64 oracle beside it on
    the whole workload (it is small enough), and parity on that output."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import MeetForward
    from workloads import MEET_WORKLOADS, make_meet_inputs
    w = MEET_WORKLOADS["meet_chain_2048"]
    inp = make_meet_inputs(w)
    d = w.dims()
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(torch.bfloat16).to(dev) for k in ("q", "k", "v")}
    for k in ("x", "rho", "s"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev)
    plan = MeetForward(**d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = plan.bind(t["q"], t["k"], t["v"], t["x"], t["rho"], t["s"], stream=stream)
    for _ in range(warmup):
        plan.forward_raw(raw)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.forward_raw(raw)
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps
    pairs = d["B"] * d["L"] * d["L"]
    # algorithmic count of the pages' lifted form (MEET eq. 7-8): the query
    # and key rows carry C + 9 columns, the value rows C
    flops = 2.0 * d["H"] * (2 * d["C"] + 9) * pairs
    out = {"workload": w.name, "config": {**d, "storage": "bf16"}, "ms_per_call": ms,
           "pairs_per_s": pairs / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
           "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS,
           "executed_note": "runs on the IPA kernels with 128-wide lifted rows"}
    if cpu:
        gpu = plan.out.cpu().numpy()
        out["cpu_baseline"] = cpu["baseline"]
        out["parity_max_abs_err"] = float(np.abs(gpu.astype(np.float64) - cpu["ref"]).max())
    return out


def bench_frames(dev, steps: int, warmup: int, cpu) -> dict:
    """Frames from backbone atoms (ipa_frames_from_atoms) over 16 chains of
    16384 residues: bytes moved per residue (36 read, 48 written) against
    the HBM peak, and the fp64 oracle on the same atoms."""
    import ctypes
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import load_library
    from workloads import make_backbone
    B, L = 16, 16384
    bb = make_backbone(B, L, seed=0)
    t = {k: torch.from_numpy(v).to(dev) for k, v in bb.items()}
    rot = torch.empty(B, L, 3, 3, dtype=torch.float32, device=dev)
    trans = torch.empty(B, L, 3, dtype=torch.float32, device=dev)
    lib = load_library()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    args = (B, L, t["n"].data_ptr(), t["ca"].data_ptr(), t["c"].data_ptr(), rot.data_ptr(), trans.data_ptr(), sp)
    for _ in range(warmup):
        lib.ipa_frames_from_atoms(*args)
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        rc = lib.ipa_frames_from_atoms(*args)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    assert rc == 0
    ms = ev[0].elapsed_time(ev[1]) / steps
    nbytes = B * L * (36 + 48)
    out = {"workload": f"backbone B={B} L={L}", "ms_per_call": ms, "residues_per_s": B * L / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "algorithmic_bytes": nbytes}}
    if cpu:
        out["cpu_baseline"] = cpu["baseline"]
        out["parity_max_abs_err"] = float(np.abs(rot.cpu().numpy().astype(np.float64) - cpu["ref"]).max())
    return out


def dirdist_valu_flops_per_triple() -> int:
    """Algorithmic fp32 vector operations per (query, key, head) of the
    direction-and-distance attention's logit and softmax, each counted once:
    direction dot 5, point difference 3, squared norm 5, square root 1, the
    logit's scale-and-subtract 2, running-max compare 1, subtract +
    exponential + sum 3."""
    return 20


def dirdist_mfma_flops_per_triple(M: int) -> int:
    """The weighted sum of the 3M rotated value coordinates per (query, key,
    head): one multiply and one add each, run on the matrix cores."""
    return 6 * M


def bench_dirdist(dev, steps: int, warmup: int, cpu) -> dict:
    """Direction-and-distance attention (ipa_dirdist_forward) on the
    2048-residue chain, vectors and readout (no attention matrix): the whole
    forward timed like the IPA step, its vector-ALU roofline with the matrix
    part reported apart, and parity on the oracle's sampled rows."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import DirDistForward
    from workloads import DIRDIST_WORKLOADS, make_dirdist_inputs
    w = DIRDIST_WORKLOADS["dd_chain_2048"]
    inp = make_dirdist_inputs(w)
    d = w.dims()
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in DD_NAMES}
    fm = torch.from_numpy(inp["frame_mask"]).to(dev)
    plan = DirDistForward(**d, device=dev, attention=False)
    stream = torch.cuda.current_stream(dev)
    raw = plan.bind(*(t[k] for k in DD_NAMES), frame_mask=fm, stream=stream)
    for _ in range(warmup):
        plan.forward_raw(raw)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.forward_raw(raw)
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        plan.forward_raw(raw)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    ev_ms = ev[0].elapsed_time(ev[1]) / steps
    triples = d["B"] * d["N"] * d["N"] * d["H"]
    valu = dirdist_valu_flops_per_triple() * triples
    mfma = dirdist_mfma_flops_per_triple(d["M"]) * triples
    ach = valu / (ev_ms * 1e-3) / 1e12
    out = {"workload": w.name, "config": {**d, "storage": "fp32"}, "ms_per_call": ms,
           "ms_per_call_events": ev_ms, "pairs_per_s": d["B"] * d["N"] * d["N"] / (ms * 1e-3),
           "roofline": {"bound": "alu", "achieved": ach, "peak": PEAK_FP32_VECTOR_TFLOPS,
                        "unit": "TFLOP/s", "frac": ach / PEAK_FP32_VECTOR_TFLOPS, "flops_per_call": valu,
                        "note": "whole forward (lift, loop, merge, readout) timed; vector fp32 operations of "
                                "the logit and softmax against the peak without packed fp32"},
           "mfma_part": {"flops_per_call": mfma, "achieved": mfma / (ev_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                         "peak": PEAK_MFMA_TFLOPS,
                         "note": "probability-weighted rotated values, run as three bf16 products on split "
                                 "fp32 operands; flops counted once"}}
    if cpu:
        vec = plan.vectors.cpu().numpy()
        outp = plan.output.cpu().numpy()
        err = 0.0
        for rows, ref in zip(cpu["rows"], cpu["refs"]):
            scale = max(1.0, float(np.abs(ref["output"]).max()))
            err = max(err, float(np.abs(vec[:, rows] - ref["vectors"]).max()),
                      float(np.abs(outp[:, rows] - ref["output"]).max()) / scale)
        out["cpu_baseline"] = cpu["baseline"]
        out["parity_max_err"] = err
    return out


def backward_flops_per_pair(d: dict) -> int:
    """Algorithmic fp32 operations of the gradient per (query, key, head),
    each product or sum counted once: the logit's lifted dot (2 DA) and point
    term (3 per coordinate + 2), dP (2 DV), the softmax and dS (4), then
    dS KA' (2 (DA + 3Pqk)), A z2 (2 R Cz), dS^T QA' (2 (DA + 3Pqk + 1)),
    A^T GA (2 DV) and the gamma term (2)."""
    DA = d["C"] + d["R"] * d["Cz"]
    DV = d["C"] + 3 * d["Pv"] + d["R"] * d["Cz"]
    P3 = 3 * d["Pqk"]
    return (2 * DA + 3 * P3 + 2 + 2 * DV + 4 + 2 * (DA + P3) + 2 * d["R"] * d["Cz"]
            + 2 * (DA + P3 + 1) + 2 * DV + 2)


def bench_backward(dev, steps: int, warmup: int, cpu, flash: bool = False) -> dict:
    """Gradient of the IPA forward at the long_chain_2048 dimensions:
    ipa_backward (float32 features, score rows of a query chunk stored) or,
    with ``flash``, ipa_backward_flash (bf16 features, no score rows). The
    forward outputs come from the forward kernels on the same inputs, the
    cotangents are N(0, 1). Timed between HIP events over back-to-back
    calls; the fp64 oracle is timed on a 256-residue chain of the same
    dimensions and scaled per pair."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import IPABackward, IPABackwardFlash, IPAForward
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[HEADLINE]
    inp = make_inputs(w)
    d = w.dims()
    names = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "w_b", "gamma")
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(dev) for n in names}
    fwd = IPAForward(**d, dtype=torch.bfloat16, device=dev)
    out = fwd(*(t[n].to(torch.bfloat16) if n not in ("rot", "trans", "w_b", "gamma") else t[n] for n in names),
              w_L=inp["w_L"], w_C=inp["w_C"])
    rng = np.random.default_rng(5)
    g = {"s": (d["B"], d["L"], d["H"], d["C"]), "pts": (d["B"], d["L"], d["H"], d["Pv"], 3),
         "pts_norm": (d["B"], d["L"], d["H"], d["Pv"]), "pair": (d["B"], d["L"], d["H"], d["Cz"])}
    g = {k: torch.from_numpy(rng.standard_normal(v).astype(np.float32)).to(dev) for k, v in g.items()}
    if flash:
        bwd = IPABackwardFlash(**d, dtype=torch.bfloat16, device=dev)
        t = {n: (x.to(torch.bfloat16) if n in IPABackwardFlash._FEATURES else x) for n, x in t.items()}
    else:
        bwd = IPABackward(**d, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = bwd.bind(t, {"s": out["s"], "pts": out["pts"], "pair": out["pair"]}, g,
                   w_L=inp["w_L"], w_C=inp["w_C"], stream=stream)
    nw = max(3, warmup // 20)
    for _ in range(nw):
        bwd.backward_raw(raw)
    torch.cuda.synchronize(dev)
    n = max(10, steps // 10)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(n):
        bwd.backward_raw(raw)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    ms = ev[0].elapsed_time(ev[1]) / n
    pairs = d["B"] * d["L"] * d["L"]
    flops = backward_flops_per_pair(d) * pairs * d["H"]
    ach = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS if flash else PEAK_FP32_MFMA_TFLOPS
    res = {"workload": w.name, "config": {**d, "storage": "bf16" if flash else "fp32"},
           "form": "flash (no score rows)" if flash else "query chunks (score rows stored)",
           "calls": n, "ms_per_call": ms,
           "pairs_per_s": pairs / (ms * 1e-3), "workspace_MB": bwd.ws_bytes / 2 ** 20,
           "roofline": {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                        "frac": ach / peak, "flops_per_call": flops,
                        "note": "whole gradient timed; flops counted once per product, peak taken as "
                                + ("bf16's" if flash else "fp32's")}}
    if cpu:
        res["cpu_baseline"] = cpu["baseline"]
    return res


def bench_layer(dev, steps: int, warmup: int, cpu) -> dict:
    """The full IPA layer (ipa_layer_forward) at the long_chain_2048
    dimensions with a 384-wide single representation, bf16 attention: the
    whole layer timed like the IPA step; the projections' and readout's
    share is the difference to the bare attention step."""
    import torch
    from geometric_invariant_attention_amd import IPALayer
    from workloads import WORKLOADS, make_layer_inputs
    w = WORKLOADS[HEADLINE]
    c_s = 384
    inp = make_layer_inputs(w, c_s=c_s)
    d = w.dims()
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in ("s", "rot", "trans", "w_in", "b_in", "w_b",
                                                       "gamma", "w_out", "b_out")}
    layer = IPALayer(**d, c_s=c_s, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = layer.bind(t["s"], t["rot"], t["trans"], t["w_in"], t["b_in"], t["w_b"], t["gamma"],
                     t["w_out"], t["b_out"], w_L=inp["w_L"], w_C=inp["w_C"], stream=stream)
    for _ in range(warmup):
        layer.forward_raw(raw)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward_raw(raw)
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps
    rows = d["B"] * d["L"]
    gemm_flops = 2.0 * rows * c_s * (layer.n_in + layer.n_out)
    res = {"workload": w.name, "config": {**d, "c_s": c_s, "storage": "bf16"}, "ms_per_call": ms,
           "pairs_per_s": d["B"] * d["L"] * d["L"] / (ms * 1e-3),
           "projection_readout_gflop": gemm_flops / 1e9}
    if cpu:
        res["cpu_baseline"] = cpu["baseline"]
    return res


def memory_sweep(dev, Ls, H=12, Cz=128):
    """Peak device memory (inputs + outputs + workspace) of one forward."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import IPAForward
    res = []
    for L in Ls:
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        g = torch.Generator(device=dev).manual_seed(0)
        bf = dict(dtype=torch.bfloat16, device=dev)
        t = dict(q=torch.randn(1, L, H, 16, generator=g, **bf), k=torch.randn(1, L, H, 16, generator=g, **bf),
                 v=torch.randn(1, L, H, 16, generator=g, **bf),
                 q_pts=torch.randn(1, L, H, 4, 3, generator=g, **bf),
                 k_pts=torch.randn(1, L, H, 4, 3, generator=g, **bf),
                 v_pts=torch.randn(1, L, H, 8, 3, generator=g, **bf),
                 z1=torch.randn(1, L, 2, Cz, generator=g, **bf) * Cz ** -0.5,
                 z2=torch.randn(1, L, 2, Cz, generator=g, **bf) * Cz ** -0.5,
                 rot=torch.eye(3, device=dev).expand(1, L, 3, 3).contiguous(),
                 trans=torch.cumsum(torch.randn(1, L, 3, generator=g, device=dev) * 2.2, dim=1),
                 w_b=torch.randn(Cz, H, generator=g, device=dev),
                 gamma=torch.ones(H, device=dev))
        plan = IPAForward(1, L, H, 16, 4, 8, 2, Cz, device=dev)
        raw = plan.bind(**t)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        plan.forward_raw(raw)
        torch.cuda.synchronize(dev)
        ms = (time.perf_counter() - t0) * 1e3
        peak = torch.cuda.max_memory_allocated(dev) - base
        res.append({"L": L, "peak_MB": peak / 2 ** 20, "workspace_MB": plan.ws_bytes / 2 ** 20,
                    "first_call_ms": ms})
        del plan, raw, t
    # least-squares y = a L^2 + b L
    A = np.array([[r["L"] ** 2, r["L"]] for r in res], dtype=np.float64)
    y = np.array([r["peak_MB"] for r in res])
    coef = np.linalg.lstsq(A, y, rcond=None)[0]
    return {"H": H, "Cz": Cz, "points": res, "fit_MB": {"a_L2": float(coef[0]), "b_L": float(coef[1])}}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only-headline", action="store_true",
                    help="time only --workload (no other sizes, entry points or memory sweep)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of fp64 oracle work for the CPU baseline (0 = skip every oracle)")
    ap.add_argument("--no-mem-sweep", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes (3 times) and exit; "
                         "a reference for hardware byte counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(heads and batch elements would shard without communication)",
              file=sys.stderr)
        return 2

    from workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    d = w.dims()
    cpu = {}
    P = cpu_workers()
    if args.cpu_budget > 0 and not args.copy_calibration:
        cpu = run_cpu_side(args, P)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))
        return 0

    # the headline's inputs and plan first, so that nothing but the launch
    # loop stands between the last other GPU measurement and its steps
    head = prepare(w, dev, inp=_CPU_INPUTS.get(w.name))
    sub, cfg_preps = {}, {}
    if not args.only_headline:
        sub["meet"] = bench_meet(dev, args.steps, args.warmup, cpu.get("meet"))
        sub["frames"] = bench_frames(dev, args.steps, 20, cpu.get("frames"))
        sub["layer"] = bench_layer(dev, args.steps, args.warmup, cpu.get("layer"))
        sub["dirdist"] = bench_dirdist(dev, args.steps, args.warmup, cpu.get("dirdist"))
        sub["backward"] = bench_backward(dev, args.steps, args.warmup, cpu.get("backward"))
        sub["backward_flash"] = bench_backward(dev, args.steps, args.warmup, cpu.get("backward"), flash=True)
        print(f"[bench] distance attention {sub['meet']['ms_per_call'] * 1e3:.1f} us, layer "
              f"{sub['layer']['ms_per_call'] * 1e3:.1f} us, gradient {sub['backward']['ms_per_call']:.3f} ms "
              f"(flash {sub['backward_flash']['ms_per_call']:.3f} ms), "
              f"direction-and-distance {sub['dirdist']['ms_per_call'] * 1e3:.1f} us", file=sys.stderr, flush=True)
        sub["configs"] = {}
        for nm in CONFIGS:
            if nm != args.workload:
                sub["configs"][nm], cfg_preps[nm] = bench_config(nm, dev, args.steps, args.warmup)

    # the headline, last among the timed GPU work
    wall, lift_ms, attn_ms = time_steps(head, args.steps, args.warmup, dev)
    inp, out = head["inp"], outputs(head)
    cfg_cpu = cpu.get("configs", {})
    for nm, prep in cfg_preps.items():
        config_parity(sub["configs"][nm], prep, cfg_cpu.get(nm))
    del cfg_preps
    fig = step_figures(w, inp, wall, args.steps, lift_ms, attn_ms)
    ar = fig["attend_roofline"]
    result = {
        "metric": METRIC,
        "value": fig["pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, **d, "storage": w.dtype,
                   "mma": "bf16 (scalar/point columns, P.V) and fp16 (pair columns of Q.K^T), fp32 accumulate"},
        "tflops": fig["tflops"],
        "pct_bf16_peak": fig["pct_bf16_peak"],
        "kernels_ms": fig["kernels_ms"],
        "roofline": {"kernel": "ipa_attend", "bound": "mfma", "achieved": ar["achieved"],
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": ar["frac"],
                     "traffic": ar["traffic"], "algorithmic_flops": ar["algorithmic_flops"]},
        "lift_GBs_algorithmic": algo_bytes(d) / (lift_ms * 1e-3) / 1e9,
    }
    if "attend_hbm_GBs_counters" in fig:
        result["attend_hbm_GBs_counters"] = fig["attend_hbm_GBs_counters"]
    print(f"[bench] {w.name}: {fig['ms_per_step'] * 1e3:.1f} us/step (lift {lift_ms * 1e3:.1f} us, "
          f"attend {attn_ms * 1e3:.1f} us), {fig['tflops']:.1f} TFLOP/s, {fig['pairs_per_s']:.3e} pairs/s",
          file=sys.stderr, flush=True)

    if "headline" in cpu:
        hc = cpu["headline"]
        result["cpu_baseline"] = hc["baseline"]
        result["parity_on_cpu_sample"] = {"rows": int(sum(len(r) for r in hc["rows"])),
                                          "max_abs_err": parity_on_rows(out, hc["rows"], hc["refs"]),
                                          "tol": 3e-2 if w.dtype == "bf16" else 1e-4}
    else:
        result["cpu_baseline"] = None
    if "single_thread" in cpu:
        result["cpu_baseline_single_thread"] = cpu["single_thread"]
    result.update(sub)

    if not (args.no_mem_sweep or args.only_headline):
        result["memory_vs_L"] = memory_sweep(dev, [512, 1024, 2048, 4096, 8192, 16384])
        print(f"[bench] memory fit {result['memory_vs_L']['fit_MB']}", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
