#!/usr/bin/env python3
"""Benchmark of the fused IPA forward on one MI355X.

One step = one full forward over one batch: ipa_lift (frames -> lifted
operands) followed by ipa_attend (fused online-softmax attention + output
epilogue), on inputs already resident in device memory.

Prints ONE JSON line: throughput in residue pairs per second (all heads, the
whole job), achieved TFLOP/s against the algorithmic count
2 H (d_qk + d_v) sum_b n_b^2 with d_qk = C + 3 Pqk + 2 + R Cz and
d_v = C + 3 Pv + R Cz, the roofline of the dominant kernel (ipa_attend)
from HIP events recorded on its own stream, peak device memory versus L,
and the fp64 CPU oracle timed on a bounded row sample as a reported
baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# MI355X fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed
# fp32) x 2.4 GHz. Code built without packed fp32 issues at most half of it.
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_FP32_MFMA_TFLOPS = 157.3    # MI355X dense fp32 matrix peak
METRIC = "IPA fwd pairs/s & TFLOP/s (% bf16 MFMA peak) at L=2048; peak HBM GB vs L"


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
# FETCH_SIZE pass, one WRITE_SIZE pass) and committed as a summary together
# with the hash of the kernel source they were taken on.
PROFILE_PMC = os.path.join(ROOT, "profiles", "ipa_attend_long_chain_2048_pmc.md")
KERNEL_SOURCES = ("ipa_attn.hip", "ipa_internal.h", "ipa_api.cpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "geometric_invariant_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes of one ipa_attend launch from the committed counter summary
    (each counter scaled by what it reads for a plain copy of known size), or
    None when the summary was taken on another workload or on kernel source
    that has changed since."""
    try:
        with open(PROFILE_PMC) as fh:
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


def run_timed(w, steps: int, warmup: int, dev):
    import torch
    from geometric_invariant_attention_amd import IPAForward
    from workloads import make_inputs

    inp = make_inputs(w)
    t = to_device(inp, dev)
    d = w.dims()
    plan = IPAForward(**d, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = plan.bind(**{k: t[k] for k in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans",
                                          "z1", "z2", "w_b", "gamma")},
                    mask=t["mask"], w_L=inp["w_L"], w_C=inp["w_C"], stream=stream)
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
    lift_ms = ev[0].elapsed_time(ev[1]) / steps
    attn_ms = ev[2].elapsed_time(ev[3]) / steps
    out = {k: v.detach().cpu().numpy() for k, v in plan.out.items()}
    return inp, wall, lift_ms, attn_ms, out


def cpu_baseline(inp, gpu_out, budget_s: float):
    """Time the fp64 oracle on a bounded sample of query rows (every row is
    independent) and compare the GPU output on those rows."""
    import numpy as np
    from oracle import ipa_forward as oracle_forward

    d = inp["dims"]
    L, B = d["L"], d["B"]
    rng = np.random.default_rng(1234)
    order = rng.permutation(L)
    done, rows_all, spent_wall, spent_cpu = 0, [], 0.0, 0.0
    errs = {}
    n = 16
    while done < L and spent_wall < budget_s:
        rows = np.sort(order[done:done + n])
        c0, w0 = time.process_time(), time.perf_counter()
        ref = oracle_forward(inp, rows=rows)
        spent_wall += time.perf_counter() - w0
        spent_cpu += time.process_time() - c0
        for k in ref:
            e = float(np.abs(gpu_out[k][:, rows].astype(np.float64) - ref[k]).max())
            errs[k] = max(errs.get(k, 0.0), e)
        done += len(rows)
        rows_all.append(rows)
        n = min(2 * n, 256)
    pairs = B * done * L
    cores = max(1, round(spent_cpu / max(spent_wall, 1e-9)))
    return {
        "value": pairs / spent_wall, "unit": "pairs/s", "cores": cores, "kind": "oracle",
        "sample": f"{done} of {L} query rows x {L} keys x B={B} (all {d['H']} heads), "
                  f"fp64 numpy, {spent_wall:.1f} s wall",
    }, errs, done


def bench_meet(dev, steps: int, warmup: int, cpu: bool) -> dict:
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
        from oracle import meet_attention
        c0, w0 = time.process_time(), time.perf_counter()
        ref = meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"])
        wall = time.perf_counter() - w0
        cores = max(1, round((time.process_time() - c0) / max(wall, 1e-9)))
        gpu = plan.out.cpu().numpy()
        out["cpu_baseline"] = {"value": pairs / wall, "unit": "pairs/s", "cores": cores, "kind": "oracle",
                               "sample": f"the whole {w.name} workload ({d['L']} x {d['L']} pairs, {d['H']} heads)"}
        out["parity_max_abs_err"] = float(np.abs(gpu.astype(np.float64) - ref).max())
    return out


def bench_frames(dev, steps: int, warmup: int, cpu: bool) -> dict:
    """Frames from backbone atoms (ipa_frames_from_atoms) over 16 chains of
    16384 residues: bytes moved per residue (36 read, 48 written) against
    the HBM peak, and the fp64 oracle on the same atoms."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import load_library
    from workloads import make_backbone
    import ctypes
    B, L = 16, 16384
    bb = make_backbone(B, L, seed=0)
    t = {k: torch.from_numpy(v).to(dev) for k, v in bb.items()}
    rot = torch.empty(B, L, 3, 3, dtype=torch.float32, device=dev)
    trans = torch.empty(B, L, 3, dtype=torch.float32, device=dev)
    lib = load_library()
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (B, L, t["n"].data_ptr(), t["ca"].data_ptr(), t["c"].data_ptr(), rot.data_ptr(), trans.data_ptr(), sp)
    for _ in range(warmup):
        lib.ipa_frames_from_atoms(*args)
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        rc = lib.ipa_frames_from_atoms(*args)
    ev[1].record()
    torch.cuda.synchronize(dev)
    assert rc == 0
    ms = ev[0].elapsed_time(ev[1]) / steps
    nbytes = B * L * (36 + 48)
    out = {"workload": f"backbone B={B} L={L}", "ms_per_call": ms, "residues_per_s": B * L / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "algorithmic_bytes": nbytes}}
    if cpu:
        from oracle import frames_from_atoms
        c0, w0 = time.process_time(), time.perf_counter()
        r_ref, _ = frames_from_atoms(bb["n"], bb["ca"], bb["c"])
        wall = time.perf_counter() - w0
        cores = max(1, round((time.process_time() - c0) / max(wall, 1e-9)))
        out["cpu_baseline"] = {"value": B * L / wall, "unit": "residues/s", "cores": cores, "kind": "oracle",
                               "sample": f"the whole workload ({B * L} residues)"}
        out["parity_max_abs_err"] = float(np.abs(rot.cpu().numpy().astype(np.float64) - r_ref).max())
    return out


def dirdist_flops_per_triple(M: int) -> int:
    """Algorithmic fp32 operations per (query, key, head) of the
    direction-and-distance attention, each operation counted once: direction
    dot 5, point difference 3, squared norm 5, square root 1, the logit's
    scale-and-subtract 2, running-max compare 1, subtract + exponential +
    sum 3, weighted rotated values 2 * 3M."""
    return 20 + 6 * M


def bench_dirdist(dev, steps: int, warmup: int, cpu: bool) -> dict:
    """Direction-and-distance attention (ipa_dirdist_forward) on the
    2048-residue chain, vectors and readout (no attention matrix): the whole
    forward timed like the IPA step, its ALU roofline, the fp64 oracle on a
    bounded sample of query rows beside it, and parity on that sample."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import DirDistForward
    from workloads import DIRDIST_WORKLOADS, make_dirdist_inputs
    w = DIRDIST_WORKLOADS["dd_chain_2048"]
    inp = make_dirdist_inputs(w)
    d = w.dims()
    names = ("rot", "trans", "q_direction", "k_direction", "q_point", "k_point", "values",
             "direction_scale", "distance_scale", "output_weight", "output_bias")
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in names}
    fm = torch.from_numpy(inp["frame_mask"]).to(dev)
    plan = DirDistForward(**d, device=dev, attention=False)
    stream = torch.cuda.current_stream(dev)
    raw = plan.bind(*(t[k] for k in names), frame_mask=fm, stream=stream)
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
    flops = dirdist_flops_per_triple(d["M"]) * triples
    ach = flops / (ev_ms * 1e-3) / 1e12
    out = {"workload": w.name, "config": {**d, "storage": "fp32"}, "ms_per_call": ms,
           "ms_per_call_events": ev_ms, "pairs_per_s": d["B"] * d["N"] * d["N"] / (ms * 1e-3),
           "roofline": {"bound": "alu", "achieved": ach, "peak": PEAK_FP32_VECTOR_TFLOPS,
                        "unit": "TFLOP/s", "frac": ach / PEAK_FP32_VECTOR_TFLOPS,
                        "flops_per_call": flops,
                        "note": "whole forward (lift, loop, merge, readout) timed; flops of the loop"}}
    if cpu:
        from oracle import dirdist_attention
        vec = plan.vectors.cpu().numpy()
        outp = plan.output.cpu().numpy()
        rng = np.random.default_rng(7)
        order = rng.permutation(d["N"])
        done, spent, spent_cpu, n, err = 0, 0.0, 0.0, 16, 0.0
        scale = None
        while done < d["N"] and spent < 10.0:
            rows = np.sort(order[done:done + n])
            c0, w0 = time.process_time(), time.perf_counter()
            ref = dirdist_attention(**{k: inp[k] for k in names}, frame_mask=inp["frame_mask"], rows=rows)
            spent += time.perf_counter() - w0
            spent_cpu += time.process_time() - c0
            scale = max(1.0, float(np.abs(ref["output"]).max()))
            err = max(err, float(np.abs(vec[:, rows] - ref["vectors"]).max()),
                      float(np.abs(outp[:, rows] - ref["output"]).max()) / scale)
            done += len(rows)
            n = min(2 * n, 256)
        out["cpu_baseline"] = {"value": d["B"] * done * d["N"] / spent, "unit": "pairs/s",
                               "cores": max(1, round(spent_cpu / max(spent, 1e-9))), "kind": "oracle",
                               "sample": f"{done} of {d['N']} query rows x {d['N']} keys, all {d['H']} heads, "
                                         f"fp64 numpy, {spent:.1f} s wall"}
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


def bench_backward(dev, steps: int, warmup: int, cpu: bool) -> dict:
    """Gradient of the IPA forward (ipa_backward, float32) at the
    long_chain_2048 dimensions: the forward outputs come from the forward
    kernels on the same inputs (float32 copies of the bf16 workload), the
    cotangents are N(0, 1). Timed between HIP events over back-to-back
    calls; the fp64 oracle is timed on a 256-residue chain of the same
    dimensions and scaled per pair."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import IPABackward, IPAForward
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["long_chain_2048"]
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
    bwd = IPABackward(**d, device=dev)
    stream = torch.cuda.current_stream(dev)
    raw = bwd.bind(t, {"s": out["s"], "pts": out["pts"], "pair": out["pair"]}, g,
                   w_L=inp["w_L"], w_C=inp["w_C"], stream=stream)
    nw = max(2, warmup // 20)
    for _ in range(nw):
        bwd.backward_raw(raw)
    torch.cuda.synchronize(dev)
    n = max(2, steps // 10)
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
    res = {"workload": w.name, "config": {**d, "storage": "fp32"}, "calls": n, "ms_per_call": ms,
           "pairs_per_s": pairs / (ms * 1e-3),
           "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / PEAK_FP32_MFMA_TFLOPS, "flops_per_call": flops,
                        "note": "whole gradient timed (preparation, matrix-core GEMMs and a row kernel per "
                                "query chunk, chain rule); flops counted once per product; U, dVA and the "
                                "scalar and pair columns of dQA' run as three bf16 products on split "
                                "fp32 operands, the rest as fp32 products, peak taken as fp32's"}}
    if cpu:
        from oracle import ipa_backward as oracle_backward
        ws = w.with_(L=256)
        ci = make_inputs(ws)
        cg = {k: np.random.default_rng(1).standard_normal(
            (ws.B, ws.L) + tuple(v.shape[2:])) for k, v in g.items()}
        c0, w0 = time.process_time(), time.perf_counter()
        oracle_backward(ci, cg)
        wall = time.perf_counter() - w0
        res["cpu_baseline"] = {"value": ws.B * ws.L * ws.L / wall, "unit": "pairs/s",
                               "cores": max(1, round((time.process_time() - c0) / max(wall, 1e-9))),
                               "kind": "oracle",
                               "sample": f"fp64 autograd oracle on a {ws.L}-residue chain with the same H, C, "
                                         f"points and pair factors, {wall:.1f} s wall, scaled per pair"}
    return res


def bench_layer(dev, steps: int, warmup: int, cpu: bool) -> dict:
    """The full IPA layer (ipa_layer_forward) at the long_chain_2048
    dimensions with a 384-wide single representation, bf16 attention: the
    whole layer timed like the IPA step; the projections' and readout's
    share is the difference to the bare attention step."""
    import numpy as np
    import torch
    from geometric_invariant_attention_amd import IPALayer
    from workloads import WORKLOADS, make_layer_inputs
    w = WORKLOADS["long_chain_2048"]
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
    n_in = layer.n_in
    gemm_flops = 2.0 * rows * c_s * (n_in + layer.n_out)
    res = {"workload": w.name, "config": {**d, "c_s": c_s, "storage": "bf16"}, "ms_per_call": ms,
           "pairs_per_s": d["B"] * d["L"] * d["L"] / (ms * 1e-3),
           "projection_readout_gflop": gemm_flops / 1e9}
    if cpu:
        from oracle import ipa_layer
        ci = make_layer_inputs(w.with_(L=256), c_s=c_s)
        c0, w0 = time.process_time(), time.perf_counter()
        ipa_layer(ci)
        wall = time.perf_counter() - w0
        res["cpu_baseline"] = {"value": 256 * 256 / wall, "unit": "pairs/s",
                               "cores": max(1, round((time.process_time() - c0) / max(wall, 1e-9))),
                               "kind": "oracle",
                               "sample": f"fp64 layer oracle on a 256-residue chain with the same dimensions, "
                                         f"{wall:.2f} s wall, scaled per pair"}
    return res


def memory_sweep(dev, Ls, H=12, Cz=128):
    """Peak device memory (inputs + outputs + workspace) of one forward."""
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
    import numpy as np
    A = np.array([[r["L"] ** 2, r["L"]] for r in res], dtype=np.float64)
    y = np.array([r["peak_MB"] for r in res])
    coef = np.linalg.lstsq(A, y, rcond=None)[0]
    return {"H": H, "Cz": Cz, "points": res, "fit_MB": {"a_L2": float(coef[0]), "b_L": float(coef[1])}}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the clocks take a few tens of milliseconds of load to settle
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="long_chain_2048")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of fp64 oracle work for the CPU baseline (0 = skip)")
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

    import torch
    from workloads import WORKLOADS

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
    w = WORKLOADS[args.workload]
    d = w.dims()

    inp, wall, lift_ms, attn_ms, out = run_timed(w, args.steps, args.warmup, dev)
    ms_step = wall * 1e3 / args.steps
    pairs = int((inp["lengths"].astype("int64") ** 2).sum())
    flops = algo_flops(d, pairs)
    value = pairs / (ms_step * 1e-3)
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, **d, "storage": w.dtype,
                   "mma": "bf16 (scalar/point columns, P.V) and fp16 (pair columns of Q.K^T), fp32 accumulate"},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_MFMA_TFLOPS,
        "kernels_ms": {"ipa_lift": lift_ms, "ipa_attend": attn_ms},
        "roofline": {"kernel": "ipa_attend", "bound": "mfma", "achieved": attn_tflops,
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_MFMA_TFLOPS,
                     "traffic": traffic["bytes"] if traffic else None,
                     "algorithmic_flops": flops},
        "lift_GBs_algorithmic": algo_bytes(d) / (lift_ms * 1e-3) / 1e9,
    }
    if traffic:
        result["attend_hbm_GBs_counters"] = traffic["bytes"] / (attn_ms * 1e-3) / 1e9
    print(f"[bench] {w.name}: {ms_step * 1e3:.1f} us/step (lift {lift_ms * 1e3:.1f} us, "
          f"attend {attn_ms * 1e3:.1f} us), {tflops:.1f} TFLOP/s, {value:.3e} pairs/s", file=sys.stderr, flush=True)

    if args.cpu_budget > 0:
        cb, errs, rows = cpu_baseline(inp, out, args.cpu_budget)
        result["cpu_baseline"] = cb
        result["parity_on_cpu_sample"] = {"rows": rows, "max_abs_err": errs, "tol": 3e-2 if w.dtype == "bf16" else 1e-4}
        print(f"[bench] cpu baseline {cb['value']:.3e} pairs/s ({cb['sample']}); max-abs errors {errs}",
              file=sys.stderr, flush=True)
    else:
        result["cpu_baseline"] = None

    result["meet"] = bench_meet(dev, args.steps, args.warmup, args.cpu_budget > 0)
    print(f"[bench] distance attention: {result['meet']['ms_per_call'] * 1e3:.1f} us/call, "
          f"{result['meet']['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    result["frames"] = bench_frames(dev, args.steps, 20, args.cpu_budget > 0)
    print("[bench] layer", file=sys.stderr, flush=True)
    result["layer"] = bench_layer(dev, args.steps, args.warmup, args.cpu_budget > 0)
    print("[bench] backward", file=sys.stderr, flush=True)
    result["backward"] = bench_backward(dev, args.steps, args.warmup, args.cpu_budget > 0)
    print("[bench] direction-and-distance attention", file=sys.stderr, flush=True)
    result["dirdist"] = bench_dirdist(dev, args.steps, args.warmup, args.cpu_budget > 0)
    print(f"[bench] frames: {result['frames']['ms_per_call'] * 1e3:.1f} us/call, "
          f"{result['frames']['roofline']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)

    if not args.no_mem_sweep:
        result["memory_vs_L"] = memory_sweep(dev, [512, 1024, 2048, 4096, 8192, 16384])
        print(f"[bench] memory fit {result['memory_vs_L']['fit_MB']}", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
