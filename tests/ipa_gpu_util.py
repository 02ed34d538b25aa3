"""Shared helpers of the GPU tests: move seeded numpy inputs onto the device
and compare the HIP outputs with the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

FEATS = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2")
FRAMES = ("rot", "trans", "w_b", "gamma")
OUTS = ("s", "pts", "pts_norm", "pair")


def to_device(inp: dict, device) -> dict:
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dt).to(device) for k in FEATS}
    for k in FRAMES:
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(device)
    t["mask"] = torch.from_numpy(inp["mask"]).to(device) if inp.get("has_mask") else None
    t["w_L"], t["w_C"] = inp["w_L"], inp["w_C"]
    return t


def run_gpu(dev_inp: dict) -> dict:
    from geometric_invariant_attention_amd import ipa_forward
    args = {k: dev_inp[k] for k in FEATS + FRAMES}
    out = ipa_forward(**args, mask=dev_inp["mask"], w_L=dev_inp["w_L"], w_C=dev_inp["w_C"])
    torch.cuda.synchronize()
    return {k: out[k].detach().cpu().numpy().copy() for k in OUTS}


def compare(gpu: dict, ref: dict, tol: float, valid_rows=None, rows=None) -> dict:
    """Max-abs error per output over valid rows (optionally only `rows`)."""
    errs = {}
    for k in OUTS:
        g = gpu[k] if rows is None else gpu[k][:, rows]
        r = ref[k]
        if valid_rows is not None:
            vr = valid_rows if rows is None else valid_rows[:, rows]
            g, r = g[vr], r[vr]
        assert np.all(np.isfinite(g)), f"{k}: non-finite values"
        errs[k] = float(np.max(np.abs(g.astype(np.float64) - r))) if g.size else 0.0
    bad = {k: e for k, e in errs.items() if e > tol}
    assert not bad, f"max-abs errors above {tol}: {bad} (all: {errs})"
    return errs


def assert_masked_positive_zero(gpu: dict, mask: np.ndarray):
    inval = mask == 0
    for k in OUTS:
        sel = np.ascontiguousarray(gpu[k][inval])
        bits = sel.view(np.uint32)
        assert np.all(bits == 0), f"{k}: masked rows are not +0.0"
