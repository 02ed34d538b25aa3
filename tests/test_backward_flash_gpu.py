"""GPU parity of the flash-form IPA gradient (ipa_backward_flash) against the
fp64 gradient oracle, through the C ABI.

The forward outputs handed to the gradient are the oracle's (rounded to
float32): a row's outputs enter only its own D_i = dO_i . O_i, and with the
oracle's outputs the test measures the gradient kernels alone.

Tolerance per gradient tensor: max-abs error <= 2e-2 x max(max |reference|,
5e-3). The floor covers tensors that vanish by cancellation (with a single
residue the translation gradient is zero; the kernels reach it to about
2^-17 of the point cotangents, which are of order 1 here). Derivation: every product of
the quadratic part takes bf16 operands, each rounded once (2^-9 relative),
times a probability or dS rounded to bf16 (2^-9), so each term carries up
to 2^-8 ~ 3.9e-3 relative error with fp32 accumulation; the sums over keys
or queries cancel (dS sums to zero over a row), which scales the error
relative to the result by the ratio sum|term| / |sum|, a few units on these
inputs. 2e-2 is five times the per-term bound; the bf16 forward's own bar is
3e-2.
"""

import numpy as np
import pytest
import torch

from oracle import ipa_backward as oracle_backward
from oracle import ipa_forward as oracle_forward
from workloads import WORKLOADS, make_inputs, stress_pair

pytestmark = pytest.mark.gpu

TOL = 2e-2
FLOOR = 5e-3
NAMES = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "w_b", "gamma")
FEATURES = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2")


def _cotangents(inp, seed):
    d = inp["dims"]
    rng = np.random.default_rng(seed)
    B, L, H = d["B"], d["L"], d["H"]
    return {"s": rng.standard_normal((B, L, H, d["C"])).astype(np.float32),
            "pts": rng.standard_normal((B, L, H, d["Pv"], 3)).astype(np.float32),
            "pts_norm": rng.standard_normal((B, L, H, d["Pv"])).astype(np.float32),
            "pair": rng.standard_normal((B, L, H, d["Cz"])).astype(np.float32)}


def _flash(inp, outs, g, device, dtype):
    from geometric_invariant_attention_amd import IPABackwardFlash
    d = inp["dims"]
    t = {}
    for n in NAMES:
        x = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(device)
        t[n] = x.to(dtype) if n in FEATURES else x
    m = torch.from_numpy(inp["mask"]).to(device) if inp.get("has_mask") else None
    o = {k: torch.from_numpy(np.ascontiguousarray(outs[k], dtype=np.float32)).to(device) for k in ("s", "pts", "pair")}
    gt = {k: torch.from_numpy(v).to(device) for k, v in g.items()}
    bwd = IPABackwardFlash(**d, dtype=dtype, device=device)
    grads = bwd(t, o, gt, mask=m, w_L=inp["w_L"], w_C=inp["w_C"])
    torch.cuda.synchronize()
    return {n: grads[n].cpu().numpy().copy() for n in NAMES}


def _errs(got, ref):
    errs = {}
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
        scale = max(float(np.abs(ref[n]).max()), FLOOR)
        err = float(np.abs(got[n] - ref[n]).max())
        errs[n] = err / scale
        assert err <= TOL * scale, (n, err, scale)
    return errs


def _check(w, device, seed=0, stress=False, dtype=torch.bfloat16):
    print(f"[flash backward] {w.name} dims={w.dims()} seed={seed} stress={stress} {dtype}", flush=True)
    inp = make_inputs(w, seed=seed)
    if stress:
        inp = stress_pair(inp)
    g = _cotangents(inp, seed + 100)
    outs = oracle_forward(inp)
    got = _flash(inp, outs, g, device, dtype)
    ref = oracle_backward(inp, g)
    errs = _errs(got, ref)
    print("  rel errors", {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    return inp, got, ref


@pytest.mark.parametrize("L", [1, 7, 33, 64, 100])
def test_flash_backward_small_fp32_storage(device, L):
    """Lengths below, at and across the 32-row block and 64-row tile, with a
    ragged tail; float32 storage of the features."""
    _check(WORKLOADS["tiny_fp32"].with_(L=L, H=3), device, seed=L, dtype=torch.float32)


@pytest.mark.parametrize("L", [5, 64, 130])
def test_flash_backward_small_bf16_storage(device, L):
    _check(WORKLOADS["tiny_fp32"].with_(L=L, H=3, dtype="bf16"), device, seed=L + 1)


def test_flash_backward_full_width_rows(device):
    """The widest lifted rows of the envelope: c_z = 128, R = 2 (the
    benchmark's row widths), several tiles with a ragged tail."""
    _check(WORKLOADS["single_chain"].with_(L=200, H=4), device, seed=5)


def test_flash_backward_pair_stress(device):
    _check(WORKLOADS["tiny_fp32"].with_(L=96, H=4, dtype="bf16"), device, seed=3, stress=True)


def test_flash_backward_other_shapes(device):
    """Odd widths: C, points and pair widths not multiples of 8 or 32."""
    w = WORKLOADS["tiny_fp32"].with_(L=70, H=2, C=5, Pqk=3, Pv=5, R=3, Cz=20)
    _check(w, device, seed=9, dtype=torch.float32)
    _check(w.with_(C=16, Pqk=5, Pv=8, R=1, Cz=256, L=40), device, seed=10)


def test_flash_backward_scattered_mask(device):
    """Non-prefix masks (masked first and last residues, fully masked
    64-residue blocks, lone valid residues): masked rows get +0.0."""
    w = WORKLOADS["tiny_fp32"].with_(B=3, L=300, H=2, Cz=16, mask="scatter", dtype="bf16")
    inp, got, ref = _check(w, device, seed=2)
    pad = inp["mask"] == 0
    assert pad.any()
    for n in NAMES:
        if n not in ("w_b", "gamma"):
            assert np.all(got[n][pad] == 0) and not np.signbit(got[n][pad]).any(), n


def test_flash_backward_ragged_batch(device):
    w = WORKLOADS["ragged_batch"].with_(B=4, L=128)
    _check(w, device, seed=4)


def test_flash_backward_deterministic(device):
    w = WORKLOADS["tiny_fp32"].with_(L=150, H=3, dtype="bf16")
    inp = make_inputs(w, seed=6)
    g = _cotangents(inp, 7)
    outs = oracle_forward(inp)
    a = _flash(inp, outs, g, device, torch.bfloat16)
    b = _flash(inp, outs, g, device, torch.bfloat16)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_flash_backward_long_chain_sampled_rows(device):
    """The benchmarked size (L = 2048, H = 12, c_z = 128, R = 2, bf16
    features). The outputs handed over are the bf16 forward's except on the
    sampled rows (tile and block edges and random rows), which get the
    oracle's; there dq, dq_pts and dz1 (query-side inputs that reach no
    other row's output) are compared with the row-restricted oracle. Over
    all rows, sum_j dv_j = sum_i g_s,i (every row's weights sum to 1)."""
    from geometric_invariant_attention_amd import IPAForward
    w = WORKLOADS["long_chain_2048"]
    d = w.dims()
    print(f"[flash backward] {w.name} dims={d} sampled rows", flush=True)
    inp = make_inputs(w, seed=0)
    L = w.L
    edges = {i for t in range(0, L + 1, 32) for i in (t - 1, t) if 0 <= i < L}
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set(sorted(edges)[::5]) | set(rng.choice(L, 16, replace=False).tolist())))
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(device) for n in NAMES}
    fwd = IPAForward(**d, dtype=torch.bfloat16, device=device)
    out = fwd(*(t[n].to(torch.bfloat16) if n in FEATURES else t[n] for n in NAMES),
              w_L=inp["w_L"], w_C=inp["w_C"])
    torch.cuda.synchronize()
    o = {k: out[k].float().cpu().numpy().copy() for k in ("s", "pts", "pair")}
    ref_o = oracle_forward(inp, rows=rows)
    for k in o:
        o[k][:, rows] = ref_o[k].astype(np.float32)
    g = _cotangents(inp, 31)
    got = _flash(inp, o, g, device, torch.bfloat16)
    ref = oracle_backward(inp, g, rows=rows)
    for n in ("q", "q_pts", "z1"):
        assert np.isfinite(got[n]).all(), n
        r = ref[n][:, rows]
        err = float(np.abs(got[n][:, rows] - r).max())
        scale = float(np.abs(r).max())
        print(f"  {n}: {len(rows)} rows, rel error {err / scale:.2e}", flush=True)
        assert err <= TOL * scale, (n, err, scale)
    sv = got["v"].astype(np.float64).sum(axis=1)
    sg = g["s"].astype(np.float64).sum(axis=1)
    scale = np.abs(g["s"]).astype(np.float64).sum(axis=1)
    dev = float((np.abs(sv - sg) / scale).max())
    print(f"  sum_j dv_j - sum_i g_s,i: {dev:.2e} of sum |g_s|", flush=True)
    assert dev < 1e-3, dev
