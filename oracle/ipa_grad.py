"""fp64 CPU oracle for the gradient of the IPA forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the
HIP path and imports nothing from it.

What is computed: the vector-Jacobian product of the forward defined in
``oracle/ipa_oracle.py`` ("Flash Invariant Point Attention", TL;DR and
abstract: the model is trained through this attention; MEET section 2.2
eq. 6 for the distance term): for output cotangents (g_s, g_pts, g_norm,
g_pair) it returns d<g, forward(x)>/dx for every input x: q, k, v, q_pts,
k_pts, v_pts, rot, trans, z1, z2, w_b, gamma. The forward is restated here
in torch (float64, explicit [L, L] tensors) and differentiated by autograd,
a library primitive applied to the definition; nothing is blocked, fused or
reordered.

Reading taken where the definition has no derivative: the point norm
|o_pts| is not differentiable at 0; its gradient there is taken as 0
(torch's convention for the norm at the origin). Masked rows (outputs
forced to +0.0) pass no gradient.

Pinning status (tests/test_grad_pins.py): central finite differences of
the numpy oracle ``ipa_forward`` along random directions, for every input;
the torch forward restated here equals ``ipa_forward``; rigid-motion
invariance of the loss gives zero gradient along the generators of the
global motion; the row-restricted form (``rows=``) against the full one.
"""

from __future__ import annotations

import math

import numpy as np
import torch

F64 = torch.float64
INPUTS = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "w_b", "gamma")


def _forward_torch(x: dict, mask: torch.Tensor, w_L: float, w_C: float, rows=None) -> dict:
    """The IPA forward of ``oracle.ipa_oracle.ipa_forward`` in torch fp64.

    ``rows`` (optional index array) restricts the query side to those rows
    (every key is still attended); outputs then have those rows only.
    """
    q, k, v = x["q"], x["k"], x["v"]
    rot, trans = x["rot"], x["trans"]
    B, L, H, C = q.shape
    qi = torch.arange(L) if rows is None else torch.as_tensor(np.asarray(rows, dtype=np.int64))

    def glob(pts):          # R_i x + t_i for every head and point
        return torch.einsum("blxy,blhpy->blhpx", rot, pts) + trans[:, :, None, None, :]

    Qg, Kg, Vg = glob(x["q_pts"])[:, qi], glob(x["k_pts"]), glob(x["v_pts"])
    Z = torch.einsum("birc,bjrc->bijc", x["z1"][:, qi], x["z2"])                # [B,L',L,Cz]
    bias = torch.einsum("bijc,ch->bijh", Z, x["w_b"])
    diff = Qg[:, :, None] - Kg[:, None, :]                                      # [B,L',L,H,P,3]
    dist = (diff * diff).sum(dim=(-1, -2))                                      # [B,L',L,H]
    scal = torch.einsum("bihc,bjhc->bijh", q[:, qi], k) / math.sqrt(C)
    S = w_L * (scal + bias - (x["gamma"] * w_C / 2.0) * dist)
    allowed = (mask[:, qi, None] & mask[:, None, :])[..., None]                 # [B,L',L,1]
    S = torch.where(allowed, S, torch.tensor(-math.inf, dtype=F64))
    m = S.amax(dim=2, keepdim=True)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    e = torch.where(allowed, torch.exp(S - m), torch.zeros_like(S))
    den = e.sum(dim=2, keepdim=True)
    a = e / torch.where(den > 0, den, torch.ones_like(den))                     # [B,L',L,H]
    o_s = torch.einsum("bijh,bjhc->bihc", a, v)
    og = torch.einsum("bijh,bjhpx->bihpx", a, Vg)
    rel = og - trans[:, qi, None, None, :]
    o_pts = torch.einsum("biyx,bihpy->bihpx", rot[:, qi], rel)
    # norm with a zero gradient at the origin
    sq = (o_pts * o_pts).sum(-1)
    safe = torch.where(sq > 0, sq, torch.ones_like(sq))
    o_norm = torch.where(sq > 0, torch.sqrt(safe), torch.zeros_like(sq))
    o_pair = torch.einsum("bijh,bijc->bihc", a, Z)
    keep = mask[:, qi, None]
    zero = torch.zeros((), dtype=F64)
    return {"s": torch.where(keep[..., None], o_s, zero),
            "pts": torch.where(keep[..., None, None], o_pts, zero),
            "pts_norm": torch.where(keep[..., None], o_norm, zero),
            "pair": torch.where(keep[..., None], o_pair, zero)}


def ipa_forward_torch(inp: dict) -> dict:
    """The restated forward as numpy fp64 (for the consistency pin)."""
    x = {n: torch.tensor(np.asarray(inp[n], dtype=np.float64)) for n in INPUTS}
    mask = _mask(inp)
    with torch.no_grad():
        out = _forward_torch(x, mask, float(inp["w_L"]), float(inp["w_C"]))
    return {k: v.numpy() for k, v in out.items()}


def _mask(inp: dict) -> torch.Tensor:
    d = inp["dims"]
    m = inp.get("mask")
    if m is None or not inp.get("has_mask", m is not None):
        return torch.ones((d["B"], d["L"]), dtype=torch.bool)
    return torch.tensor(np.asarray(m).astype(bool))


def ipa_backward(inp: dict, grads: dict, rows=None) -> dict:
    """Gradients of sum_o <grads[o], forward(inp)[o]> for every input.

    inp: the forward's input dict (``workloads.make_inputs`` layout);
    grads: "s" [B,L,H,C], "pts" [B,L,H,Pv,3], "pts_norm" [B,L,H,Pv],
    "pair" [B,L,H,Cz]. Returns a dict keyed like INPUTS, float64 numpy.

    With ``rows`` only those query rows' outputs enter the sum (their
    cotangents are taken from ``grads``). q, q_pts and z1 of residue i enter
    only row i's outputs, so their gradients on those rows equal the full
    gradient's there; every other returned array is a partial sum.
    """
    x = {n: torch.tensor(np.asarray(inp[n], dtype=np.float64), requires_grad=True) for n in INPUTS}
    mask = _mask(inp)
    out = _forward_torch(x, mask, float(inp["w_L"]), float(inp["w_C"]), rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows, dtype=np.int64)
    loss = sum((out[k] * torch.tensor(np.asarray(grads[k], dtype=np.float64)[:, sel])).sum()
               for k in ("s", "pts", "pts_norm", "pair"))
    g = torch.autograd.grad(loss, [x[n] for n in INPUTS], allow_unused=True)
    return {n: (gi.numpy() if gi is not None else np.zeros_like(x[n].detach().numpy()))
            for n, gi in zip(INPUTS, g)}
