"""fp64 lifted-attention form of the IPA forward (algebraic spec of the fused path).

TEST INFRASTRUCTURE ONLY (see ``oracle/ipa_oracle.py``); shares no code with
the HIP path.

It reaches the oracle's result through the lifting identity of MEET
("Scalable peptide design with memory-efficient equivariant transformers",
section 2.2, eq. 7-8: a squared distance is an inner product of augmented
query and key rows) and the factorised pair representation of "Flash
Invariant Point Attention" (TL;DR), with a tiled online softmax over key
blocks. In real arithmetic it equals ``ipa_forward`` exactly; tests hold it
to 1e-12 relative.

Per head h, with alpha = w_L / sqrt(c), kappa_h = w_L gamma_h w_C / 2 and
points taken relative to the centre c_G of their G-residue block
(A'_i = Qg_i - c_I, B'_j = Kg_j - c_J, G'_j = Vg_j - c_J, delta = c_I - c_J):

  Q_aug_i = [ alpha q_i | 2 kappa A'_i | w_L W_b[:,h] * z1_ir (r = 1..R) ]
  K_aug_j = [ k_j       | B'_j         | z2_jr (r = 1..R) ]
  V_aug_j = [ v_j       | G'_j         | z2_jr (r = 1..R) ]
  S_ij = Q_aug_i . K_aug_j + col_j(I) + row_i(J) + const_i, with
  col_j  = -kappa ( sum_p |B'_jp|^2 - 2 delta . sum_p B'_jp )
  row_i  = -kappa ( 2 delta . sum_p A'_ip + Pqk |delta|^2 )
  const_i = -kappa sum_p |A'_ip|^2  (the same for every key; it cancels)

The value points are recovered as sum_j a (G'_j + c_J), the pair output as
sum_r z1_ir * (sum_j a z2_jr). Logits are scaled by log2(e) and exponentiated
with 2^x, as a base-2 online softmax would.
"""

from __future__ import annotations

import math

import numpy as np

from .ipa_oracle import _unpack, to_global

LOG2E = 1.0 / math.log(2.0)


def block_centres(trans_b, valid_b, G):
    """Mean translation of the valid residues of each G-residue block (0 if none)."""
    L = trans_b.shape[0]
    nb = (L + G - 1) // G
    cen = np.zeros((nb, 3))
    for J in range(nb):
        sl = slice(J * G, min(L, (J + 1) * G))
        m = valid_b[sl]
        if m.any():
            cen[J] = trans_b[sl][m].mean(axis=0)
    return cen


def ipa_lifted(inp: dict, G: int = 64, centres=None) -> dict:
    (q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma, mask,
     w_L, w_C) = _unpack(inp)
    B, L, H, C = q.shape
    Pqk, Pv, R, Cz = q_pts.shape[3], v_pts.shape[3], z1.shape[2], z1.shape[3]
    alpha = w_L / math.sqrt(C)
    kappa = w_L * gamma * w_C / 2.0                      # [H]
    nb = (L + G - 1) // G

    out = {"s": np.zeros((B, L, H, C)), "pts": np.zeros((B, L, H, Pv, 3)),
           "pts_norm": np.zeros((B, L, H, Pv)), "pair": np.zeros((B, L, H, Cz))}
    for b in range(B):
        valid = mask[b]
        cen = block_centres(trans[b], valid, G) if centres is None else centres[b]
        blk = np.arange(L) // G
        c_row = cen[blk]                                  # [L,3]
        A = to_global(rot[b], trans[b], q_pts[b]) - c_row[:, None, None, :]
        Bk = to_global(rot[b], trans[b], k_pts[b]) - c_row[:, None, None, :]
        Gv = to_global(rot[b], trans[b], v_pts[b]) - c_row[:, None, None, :]
        for h in range(H):
            qa = np.concatenate(
                [alpha * q[b, :, h], 2 * kappa[h] * A[:, h].reshape(L, -1),
                 ((w_L * w_b[:, h])[None, None, :] * z1[b]).reshape(L, -1)], axis=1)
            ka = np.concatenate([k[b, :, h], Bk[:, h].reshape(L, -1),
                                 z2[b].reshape(L, -1)], axis=1)
            va = np.concatenate([v[b, :, h], Gv[:, h].reshape(L, -1),
                                 z2[b].reshape(L, -1)], axis=1)
            sumA = A[:, h].sum(axis=1)                     # [L,3]
            sumB = Bk[:, h].sum(axis=1)
            nrmB = (Bk[:, h] ** 2).sum(axis=(1, 2))        # [L]
            # online softmax over key blocks, base 2
            m = np.full(L, -np.inf)
            lsum = np.zeros(L)
            acc = np.zeros((L, va.shape[1]))
            acc_c = np.zeros((L, 3))
            for J in range(nb):
                ks = slice(J * G, min(L, (J + 1) * G))
                kv = valid[ks]
                delta = c_row - cen[J][None, :]            # [L,3]
                col = -kappa[h] * (nrmB[ks][None, :]
                                   - 2.0 * delta @ sumB[ks].T)          # [L,n]
                row = -kappa[h] * (2.0 * (delta * sumA).sum(1)
                                   + Pqk * (delta ** 2).sum(1))        # [L]
                S = (qa @ ka[ks].T + col + row[:, None]) * LOG2E
                S = np.where(kv[None, :], S, -np.inf)
                mt = np.maximum(m, S.max(axis=1))
                scale = np.where(np.isfinite(m), np.exp2(m - np.where(np.isfinite(mt), mt, 0.0)), 0.0)
                p = np.where(kv[None, :], np.exp2(S - np.where(np.isfinite(mt), mt, 0.0)[:, None]), 0.0)
                lsum = lsum * scale + p.sum(1)
                acc = acc * scale[:, None] + p @ va[ks]
                acc_c = acc_c * scale[:, None] + p.sum(1)[:, None] * cen[J][None, :]
                m = mt
            ok = valid & (lsum > 0)
            inv = np.where(ok, 1.0 / np.where(ok, lsum, 1.0), 0.0)
            o = acc * inv[:, None]
            oc = acc_c * inv[:, None]
            o_s = o[:, :C]
            og = o[:, C:C + 3 * Pv].reshape(L, Pv, 3) + oc[:, None, :]
            rel = og - trans[b][:, None, :]
            o_pts = np.einsum("iyx,ipy->ipx", rot[b], rel)
            o_pair = (z1[b] * o[:, C + 3 * Pv:].reshape(L, R, Cz)).sum(axis=1)
            keep = ok
            out["s"][b, :, h] = np.where(keep[:, None], o_s, 0.0)
            out["pts"][b, :, h] = np.where(keep[:, None, None], o_pts, 0.0)
            out["pts_norm"][b, :, h] = np.where(
                keep[:, None], np.sqrt((o_pts ** 2).sum(-1)), 0.0)
            out["pair"][b, :, h] = np.where(keep[:, None], o_pair, 0.0)
    return out
