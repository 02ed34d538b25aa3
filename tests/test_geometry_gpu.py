"""GPU parity of the frame construction and the distance-penalised attention
against the fp64 oracle, through the C ABI (ipa_frames_from_atoms,
ipa_meet_forward)."""

import numpy as np
import pytest
import torch

from oracle import frames_from_atoms as oracle_frames
from oracle import meet_attention as oracle_meet
from workloads import MEET_WORKLOADS, make_backbone, make_meet_inputs

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 3e-2


def _frames_gpu(bb, device):
    from geometric_invariant_attention_amd import frames_from_atoms
    t = {k: torch.from_numpy(v).to(device) for k, v in bb.items()}
    rot, trans = frames_from_atoms(t["n"], t["ca"], t["c"])
    torch.cuda.synchronize()
    return rot.cpu().numpy(), trans.cpu().numpy()


@pytest.mark.parametrize("B,L", [(1, 1), (2, 1000), (1, 70001)])
def test_frames_parity(device, B, L):
    print(f"[frames] B={B} L={L}", flush=True)
    bb = make_backbone(B, L, seed=L)
    rot, trans = _frames_gpu(bb, device)
    ref_rot, ref_trans = oracle_frames(bb["n"], bb["ca"], bb["c"])
    assert np.isfinite(rot).all()
    assert np.abs(rot - ref_rot).max() < 1e-5
    assert np.array_equal(trans, bb["ca"])                 # the C-alpha atoms, bit for bit
    assert np.array_equal(trans.astype(np.float64), ref_trans)


def test_frames_drive_ipa_rotation_convention(device):
    """Frames built on the GPU put C on the local first axis: R^T (C - CA)."""
    bb = make_backbone(1, 300, seed=7)
    rot, _ = _frames_gpu(bb, device)
    loc = np.einsum("blxi,blx->bli", rot.astype(np.float64), (bb["c"] - bb["ca"]).astype(np.float64))
    assert np.abs(loc[..., 1:]).max() < 1e-5
    assert np.abs(loc[..., 0] - 1.52).max() < 1e-5


def _meet_gpu(inp, device):
    from geometric_invariant_attention_amd import MeetForward
    d = inp["dims"]
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dt).to(device) for k in ("q", "k", "v")}
    for k in ("x", "rho", "s"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(device)
    m = torch.from_numpy(inp["mask"]).to(device) if inp.get("has_mask") else None
    plan = MeetForward(d["B"], d["L"], d["H"], d["C"], dtype=dt, device=device)
    out = plan(t["q"], t["k"], t["v"], t["x"], t["rho"], t["s"], mask=m)
    torch.cuda.synchronize()
    return out.cpu().numpy().copy()


def _check_meet(w, device, tol, seed=None):
    print(f"[meet] {w.name} dims={w.dims()} dtype={w.dtype} seed={seed}", flush=True)
    inp = make_meet_inputs(w, seed=seed)
    gpu = _meet_gpu(inp, device)
    ref = oracle_meet(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"],
                      inp["mask"] if inp["has_mask"] else None)
    assert np.isfinite(gpu).all()
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    assert err < tol, err
    return inp, gpu, ref


def test_meet_tiny_fp32(device):
    _check_meet(MEET_WORKLOADS["meet_tiny_fp32"], device, TOL_F32)


@pytest.mark.parametrize("L", [1, 37, 200])
def test_meet_fp32_ragged_tail(device, L):
    _check_meet(MEET_WORKLOADS["meet_tiny_fp32"].with_(L=L, H=3), device, TOL_F32, seed=L)


def test_meet_chain_512_bf16(device):
    _check_meet(MEET_WORKLOADS["meet_chain_512"], device, TOL_BF16)


@pytest.mark.parametrize("L", [70, 333])
def test_meet_bf16_ragged_tail(device, L):
    _check_meet(MEET_WORKLOADS["meet_chain_512"].with_(L=L, H=3, C=8), device, TOL_BF16, seed=L)


def test_meet_ragged_batch_masked_rows_exact_zero(device):
    inp, gpu, ref = _check_meet(MEET_WORKLOADS["meet_ragged"], device, TOL_BF16)
    pad = inp["mask"] == 0
    assert np.all(gpu[pad] == 0.0) and not np.signbit(gpu[pad]).any()


def test_meet_chain_2048_bf16(device):
    _check_meet(MEET_WORKLOADS["meet_chain_2048"], device, TOL_BF16)
