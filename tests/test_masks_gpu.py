"""GPU parity under non-prefix validity masks, through the C ABI.

The masks come from ``workloads.scatter_mask``: whole interior 64-residue
blocks masked (one of them holding a single valid residue), partially
masked blocks, masked first and last residues, a batch element masked
entirely and one with a single valid residue. Masked rows hold finite
garbage. Every path that takes a mask is checked against its fp64 oracle:
the forward (bf16 and fp32 storage), the distance attention, the full layer
and the gradient. Masked rows must be bit-exact +0.0 (gradients: exactly 0
on masked residues). Tolerances are those of each path's own parity tests.
"""

import numpy as np
import pytest
import torch

from oracle import ipa_forward as oracle_forward
from workloads import MEET_WORKLOADS, WORKLOADS, make_inputs, make_meet_inputs

from ipa_gpu_util import assert_masked_positive_zero, compare, run_gpu, to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 3e-2


def _forward(w, device, tol, seed):
    print(f"[mask] forward {w.name} B={w.B} L={w.L} H={w.H} Cz={w.Cz} {w.dtype} seed={seed}", flush=True)
    inp = make_inputs(w, seed=seed)
    gpu = run_gpu(to_device(inp, device))
    ref = oracle_forward(inp)
    errs = compare(gpu, ref, tol, valid_rows=inp["mask"].astype(bool))
    assert_masked_positive_zero(gpu, inp["mask"])
    print(f"  valid rows {inp['mask'].sum(axis=1).tolist()}, errors {errs}", flush=True)


@pytest.mark.parametrize("L", [600, 1000])
def test_forward_bf16_scattered_mask(device, L):
    """Several 128-row query blocks, a ragged row tail, skipped interior key
    blocks inside the wrapped visiting order, centring blocks with few
    valid residues."""
    w = WORKLOADS["single_chain"].with_(B=5, L=L, H=3, mask="scatter")
    _forward(w, device, TOL_BF16, seed=L)


def test_forward_bf16_scattered_mask_common_start(device):
    """L = 2600 with 320-wide rows: a head's key and value rows exceed the
    L2 share above which every query block starts its key loop at tile 0,
    so the skip list of masked interior blocks runs in that order too.
    Compared on sampled rows of every batch element (the oracle restricted
    to those rows), masked rows checked everywhere."""
    w = WORKLOADS["long_chain_2048"].with_(B=3, L=2600, H=2, mask="scatter")
    print(f"[mask] forward {w.name} B={w.B} L={w.L} H={w.H} (common start)", flush=True)
    inp = make_inputs(w, seed=26)
    gpu = run_gpu(to_device(inp, device))
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(0, w.L, 97), rng.choice(w.L, 40, replace=False), [w.L - 1]]))
    ref = oracle_forward(inp, rows=rows)
    errs = compare(gpu, ref, TOL_BF16, valid_rows=inp["mask"].astype(bool), rows=rows)
    assert_masked_positive_zero(gpu, inp["mask"])
    print(f"  {len(rows)} rows, errors {errs}", flush=True)


def test_forward_bf16_scattered_mask_narrow_rows(device):
    w = WORKLOADS["single_chain"].with_(B=4, L=520, H=2, R=1, Cz=32, mask="scatter")
    _forward(w, device, TOL_BF16, seed=7)


def test_forward_fp32_scattered_mask(device):
    w = WORKLOADS["tiny_fp32"].with_(B=5, L=560, H=3, Cz=16, mask="scatter")
    _forward(w, device, TOL_F32, seed=3)


def test_meet_scattered_mask(device):
    from geometric_invariant_attention_amd import MeetForward
    from oracle import meet_attention
    for w, tol in ((MEET_WORKLOADS["meet_chain_512"].with_(B=5, L=700, H=4, mask="scatter"), TOL_BF16),
                   (MEET_WORKLOADS["meet_tiny_fp32"].with_(B=4, L=300, H=3, mask="scatter"), TOL_F32)):
        print(f"[mask] meet {w.name} B={w.B} L={w.L} {w.dtype}", flush=True)
        inp = make_meet_inputs(w, seed=5)
        d = inp["dims"]
        dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dt).to(device) for k in ("q", "k", "v")}
        for k in ("x", "rho", "s"):
            t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(device)
        m = torch.from_numpy(inp["mask"]).to(device)
        out = MeetForward(d["B"], d["L"], d["H"], d["C"], dtype=dt, device=device)(
            t["q"], t["k"], t["v"], t["x"], t["rho"], t["s"], mask=m)
        torch.cuda.synchronize()
        gpu = out.cpu().numpy()
        ref = meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"], inp["mask"])
        valid = inp["mask"].astype(bool)
        err = float(np.abs(gpu[valid].astype(np.float64) - ref[valid]).max())
        print(f"  error {err:.2e}", flush=True)
        assert err < tol, err
        pad = ~valid
        assert np.all(gpu[pad] == 0.0) and not np.signbit(gpu[pad]).any()


def test_layer_scattered_mask(device):
    from geometric_invariant_attention_amd import IPALayer
    from oracle import ipa_layer
    from workloads import make_layer_inputs
    w = WORKLOADS["single_chain"].with_(B=4, L=400, H=4, mask="scatter")
    print(f"[mask] layer {w.name} B={w.B} L={w.L}", flush=True)
    inp = make_layer_inputs(w, c_s=128, seed=9)
    d = inp["dims"]
    t = {k: torch.from_numpy(inp[k]).to(device) for k in ("s", "rot", "trans", "w_in", "b_in", "w_b",
                                                          "gamma", "w_out", "b_out")}
    m = torch.from_numpy(inp["mask"]).to(device)
    y = IPALayer(**d, c_s=128, dtype=torch.bfloat16, device=device)(
        t["s"], t["rot"], t["trans"], t["w_in"], t["b_in"], t["w_b"], t["gamma"], t["w_out"], t["b_out"],
        mask=m, w_L=inp["w_L"], w_C=inp["w_C"])
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    ref = ipa_layer(inp)
    err = float(np.abs(got - ref).max()) / max(1.0, float(np.abs(ref).max()))
    print(f"  rel error {err:.2e}", flush=True)
    assert err < 3e-2, err
    pad = inp["mask"] == 0
    assert np.all(got[pad] == 0) and not np.signbit(got[pad]).any()


def test_backward_scattered_mask(device):
    from test_backward_gpu import NAMES, _cotangents, _gpu_backward
    from oracle import ipa_backward as oracle_backward
    w = WORKLOADS["tiny_fp32"].with_(B=5, L=300, H=2, Cz=16, mask="scatter")
    print(f"[mask] backward {w.name} B={w.B} L={w.L}", flush=True)
    inp = make_inputs(w, seed=2)
    g = _cotangents(inp, 77)
    got = _gpu_backward(inp, g, device)
    ref = oracle_backward(inp, g)
    pad = inp["mask"] == 0
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
        err = float(np.abs(got[n] - ref[n]).max()) / max(1.0, float(np.abs(ref[n]).max()))
        assert err < 2e-4, (n, err)
        if n not in ("w_b", "gamma"):
            assert np.all(got[n][pad] == 0), n
