"""Pins of the IPA gradient oracle (CPU only).

The gradient oracle (oracle/ipa_grad.py) restates the forward in torch and
differentiates it with autograd. It is pinned to things other than itself:
  * its restated forward equals the numpy forward oracle;
  * central finite differences of the numpy forward oracle, along random
    directions, match <gradient, direction> for every input tensor;
  * rigid-motion invariance of the loss: moving every frame by one global
    rotation and translation changes no output, so the gradients of the
    frames satisfy sum_i dtrans_i = 0 and sum_i (drot_i R_i^T + dtrans_i t_i^T)
    is symmetric;
  * masked rows pass no gradient, masked keys receive none.
"""

import numpy as np
import pytest

from oracle import ipa_forward
from oracle.ipa_grad import INPUTS, ipa_backward, ipa_forward_torch
from workloads import WORKLOADS, make_inputs

TINY = WORKLOADS["tiny_fp32"].with_(L=7, H=2, C=4, Pqk=2, Pv=3, R=2, Cz=8)
RAGGED = WORKLOADS["ragged_batch"].with_(B=2, L=9, H=2, C=4, Pqk=2, Pv=2, R=1, Cz=8,
                                         ragged=(5, 9), dtype="fp32")


def _grads(inp, seed):
    d = inp["dims"]
    rng = np.random.default_rng(seed)
    B, L, H = d["B"], d["L"], d["H"]
    return {"s": rng.standard_normal((B, L, H, d["C"])),
            "pts": rng.standard_normal((B, L, H, d["Pv"], 3)),
            "pts_norm": rng.standard_normal((B, L, H, d["Pv"])),
            "pair": rng.standard_normal((B, L, H, d["Cz"]))}


def _loss(inp, g):
    out = ipa_forward(inp)
    return sum(float(np.sum(out[k] * g[k])) for k in ("s", "pts", "pts_norm", "pair"))


@pytest.mark.parametrize("w", [TINY, RAGGED])
def test_restated_forward_matches_numpy_oracle(w):
    inp = make_inputs(w, seed=3)
    a, b = ipa_forward(inp), ipa_forward_torch(inp)
    for k in a:
        assert np.abs(a[k] - b[k]).max() < 1e-12, k


@pytest.mark.parametrize("w,seed", [(TINY, 0), (TINY, 1), (RAGGED, 2)])
def test_finite_differences_every_input(w, seed):
    inp = make_inputs(w, seed=seed)
    for n in INPUTS:
        inp[n] = inp[n].astype(np.float64)
    g = _grads(inp, seed + 10)
    grad = ipa_backward(inp, g)
    rng = np.random.default_rng(seed + 20)
    for n in INPUTS:
        v = rng.standard_normal(inp[n].shape)
        eps = 1e-6
        plus, minus = dict(inp), dict(inp)
        plus[n] = inp[n] + eps * v
        minus[n] = inp[n] - eps * v
        fd = (_loss(plus, g) - _loss(minus, g)) / (2 * eps)
        an = float(np.sum(grad[n] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)


def test_rigid_motion_invariance_of_frame_gradients():
    inp = make_inputs(TINY.with_(B=1, L=6), seed=5)
    g = _grads(inp, 6)
    grad = ipa_backward(inp, g)
    R = inp["rot"].astype(np.float64)[0]
    t = inp["trans"].astype(np.float64)[0]
    dR, dt = grad["rot"][0], grad["trans"][0]
    assert np.abs(dt.sum(axis=0)).max() < 1e-9
    M = np.einsum("lab,lcb->ac", dR, R) + np.einsum("la,lc->ac", dt, t)
    assert np.abs(M - M.T).max() < 1e-9 * max(1.0, np.abs(M).max())


def test_masked_rows_and_keys():
    inp = make_inputs(RAGGED, seed=7)
    g = _grads(inp, 8)
    grad = ipa_backward(inp, g)
    pad = inp["mask"] == 0
    assert pad.any()
    for n in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2"):
        assert np.all(grad[n][pad] == 0), n


@pytest.mark.parametrize("w,rows", [(TINY, [0, 3, 6]), (RAGGED, [1, 5, 8])])
def test_row_restricted_query_side_matches_full(w, rows):
    """q, q_pts and z1 of residue i enter only row i's outputs: the
    row-restricted gradient equals the full one on those rows, and the
    row-restricted forward equals the numpy oracle's sampled rows."""
    inp = make_inputs(w, seed=7)
    for n in INPUTS:
        inp[n] = inp[n].astype(np.float64)
    g = _grads(inp, 17)
    full = ipa_backward(inp, g)
    part = ipa_backward(inp, g, rows=rows)
    for n in ("q", "q_pts", "z1"):
        assert np.abs(part[n][:, rows] - full[n][:, rows]).max() < 1e-12, n
    # the other rows of a query-side input get nothing from the sampled rows
    others = [i for i in range(w.L) if i not in rows]
    assert np.all(part["q"][:, others] == 0)
    import torch
    from oracle.ipa_grad import _forward_torch, _mask
    x = {n: torch.tensor(inp[n]) for n in INPUTS}
    with torch.no_grad():
        sub = _forward_torch(x, _mask(inp), float(inp["w_L"]), float(inp["w_C"]), rows=rows)
    ref = ipa_forward(inp, rows=np.asarray(rows))
    for k in ref:
        assert np.abs(sub[k].numpy() - ref[k]).max() < 1e-12, k


@pytest.mark.parametrize("w,cuts", [(TINY, [0, 2, 3, TINY.L]), (RAGGED, [0, 4, 5, RAGGED.L])])
def test_row_block_partition_sums_to_full_gradient(w, cuts):
    """Every output row enters the loss once, so the gradient is the sum of
    the row-restricted gradients over any partition of the rows into
    blocks: for every input, key-side, frame and weight gradients
    included."""
    inp = make_inputs(w, seed=23)
    for n in INPUTS:
        inp[n] = inp[n].astype(np.float64)
    g = _grads(inp, 29)
    full = ipa_backward(inp, g)
    acc = {n: np.zeros_like(full[n]) for n in INPUTS}
    for r0, r1 in zip(cuts[:-1], cuts[1:]):
        part = ipa_backward(inp, g, rows=np.arange(r0, r1))
        for n in INPUTS:
            acc[n] += part[n]
    for n in INPUTS:
        scale = max(1.0, float(np.abs(full[n]).max()))
        assert np.abs(acc[n] - full[n]).max() <= 1e-12 * scale, n
