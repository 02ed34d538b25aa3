"""fp64 CPU oracle for the invariant point attention (IPA) forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the
HIP path and imports nothing from it.

What is computed (plain definition, explicit O(L^2) tensors, numpy float64):

Sources. "Flash Invariant Point Attention" (arXiv 2505.11580), TL;DR and
abstract: IPA attends over scalar, point and pair channels, uses a factorized
pair representation z_ij built from per-residue factors z^1_i and z^2_j, and
must stay SE(3)-invariant. "Scalable peptide design with memory-efficient
equivariant transformers" (MEET), section 2.2, eq. 6: an attention logit may
carry an invariant penalty proportional to a squared distance between points
in the global frame. "Geometric direction-and-distance attention" (BioTorch),
Required behavior: rotation[B,N,3,3] maps local column vectors to the global
frame, translation[B,N,3] is the frame origin, an edge is allowed when both
frames are valid, the softmax is taken over allowed keys only, all-masked
rows give exact zeros, and aggregated vectors are taken back with R_i^T.
The IPA logit itself is not printed on the pages; its constants follow the
original IPA formulation (reading documented with the build):

  Qg_ihp = R_i q_ihp + t_i,  Kg_jhp = R_j k_jhp + t_j,  Vg_jhp = R_j v_jhp + t_j
  Z_ij   = sum_r z1_ir * z2_jr                              (elementwise, c_z)
  b_ijh  = sum_c Z_ijc W_b[c, h]
  d_ijh  = sum_p || Qg_ihp - Kg_jhp ||^2                    (from differences)
  S_ijh  = w_L ( q_ih . k_jh / sqrt(c) + b_ijh - gamma_h w_C / 2 * d_ijh )
  a_ijh  = softmax over allowed j of S_ijh (0 outside the allowed set)
  o_s    = sum_j a v_jh
  o_pts  = R_i^T ( sum_j a Vg_jhp - t_i )
  o_norm = || o_pts ||   (plain Euclidean norm, no epsilon)
  o_pair = sum_j a Z_ij
  rows whose own frame is invalid: all four outputs are +0.0.

Each function below cites the passage it follows.
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


def _unpack(inp):
    d = inp["dims"]
    mask = inp.get("mask")
    if mask is None:
        mask = np.ones((d["B"], d["L"]), dtype=np.uint8)
    return (
        _f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"]),
        _f64(inp["q_pts"]), _f64(inp["k_pts"]), _f64(inp["v_pts"]),
        _f64(inp["rot"]), _f64(inp["trans"]),
        _f64(inp["z1"]), _f64(inp["z2"]),
        _f64(inp["w_b"]), _f64(inp["gamma"]),
        np.asarray(mask).astype(bool),
        float(inp["w_L"]), float(inp["w_C"]),
    )


def to_global(rot_b, trans_b, pts_b):
    """Apply frames T_i = (R_i, t_i) to local points: R_i x + t_i.

    "Geometric direction-and-distance attention", Required behavior: the
    rotation maps local column vectors to the global frame and the translation
    is the global origin. rot_b [L,3,3], trans_b [L,3], pts_b [L,H,P,3].
    """
    return np.einsum("lxy,lhpy->lhpx", rot_b, pts_b) + trans_b[:, None, None, :]


def ipa_forward(inp: dict, rows=None, row_block: int | None = None) -> dict:
    """Explicit O(L^2) IPA forward in fp64; see the module docstring.

    ``rows`` (optional 1-D int array) restricts the computation to those query
    rows of every batch element (each query row is independent); outputs then
    have L' = len(rows) along the residue axis.

    Returns dict with "s" [B,L',H,C], "pts" [B,L',H,Pv,3],
    "pts_norm" [B,L',H,Pv], "pair" [B,L',H,Cz] (float64).
    """
    (q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma, mask,
     w_L, w_C) = _unpack(inp)
    B, L, H, C = q.shape
    Pv = v_pts.shape[3]
    Cz = z1.shape[3]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    n_rows = len(rows)
    if row_block is None:
        # bound the explicit [rows, L, ...] temporaries to roughly 256 MB
        per_row = L * (Cz + 2 * H * 12 + 4 * H) * 8
        row_block = max(1, min(256, (256 << 20) // max(per_row, 1)))

    out_s = np.zeros((B, n_rows, H, C))
    out_pts = np.zeros((B, n_rows, H, Pv, 3))
    out_norm = np.zeros((B, n_rows, H, Pv))
    out_pair = np.zeros((B, n_rows, H, Cz))

    for b in range(B):
        # Step 1: global points (frames applied to every head's points).
        Qg = to_global(rot[b], trans[b], q_pts[b])   # [L,H,Pqk,3]
        Kg = to_global(rot[b], trans[b], k_pts[b])
        Vg = to_global(rot[b], trans[b], v_pts[b])   # [L,H,Pv,3]
        valid = mask[b]
        for s0 in range(0, n_rows, row_block):
            ridx = rows[s0:s0 + row_block]
            sl = slice(s0, s0 + len(ridx))
            # Step 2: explicit pair tensor from the rank-R factors
            # (FlashIPA TL;DR: factorized pair representation z_ij).
            Z = np.einsum("irc,jrc->ijc", z1[b, ridx], z2[b])          # [r,L,Cz]
            # Step 3: pair bias through the supplied per-head projection.
            bias = np.einsum("ijc,ch->ijh", Z, w_b)                     # [r,L,H]
            # Step 4: squared point distances, from explicit differences.
            diff = Qg[ridx][:, None] - Kg[None, :]                      # [r,L,H,P,3]
            dist = np.einsum("ijhpx,ijhpx->ijh", diff, diff)
            # Step 5: logits.
            scal = np.einsum("ihc,jhc->ijh", q[b, ridx], k[b]) / math.sqrt(C)
            S = w_L * (scal + bias - (gamma * w_C / 2.0)[None, None, :] * dist)
            # Step 6: softmax over allowed keys only; empty rows stay zero
            # ("Geometric direction-and-distance attention", Required behavior).
            allowed = valid[ridx][:, None] & valid[None, :]             # [r,L]
            S = np.where(allowed[:, :, None], S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(allowed[:, :, None], np.exp(S - m), 0.0)
            den = e.sum(axis=1, keepdims=True)
            a = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)  # [r,L,H]
            # Step 7: outputs.
            o_s = np.einsum("ijh,jhc->ihc", a, v[b])
            og = np.einsum("ijh,jhpx->ihpx", a, Vg)
            rel = og - trans[b, ridx][:, None, None, :]
            # R_i^T y: (R^T y)_x = sum_y R[y, x] y_y
            o_pts = np.einsum("iyx,ihpy->ihpx", rot[b, ridx], rel)
            o_norm = np.sqrt(np.einsum("ihpx,ihpx->ihp", o_pts, o_pts))
            o_pair = np.einsum("ijh,ijc->ihc", a, Z)
            # Step 8: rows with an invalid frame output +0.0 everywhere.
            keep = valid[ridx]
            out_s[b, sl] = np.where(keep[:, None, None], o_s, 0.0)
            out_pts[b, sl] = np.where(keep[:, None, None, None], o_pts, 0.0)
            out_norm[b, sl] = np.where(keep[:, None, None], o_norm, 0.0)
            out_pair[b, sl] = np.where(keep[:, None, None], o_pair, 0.0)

    # make every zero a positive zero
    for o in (out_s, out_pts, out_norm, out_pair):
        o += 0.0
    return {"s": out_s, "pts": out_pts, "pts_norm": out_norm, "pair": out_pair}
