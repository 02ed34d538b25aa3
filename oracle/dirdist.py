"""fp64 CPU oracle for geometric direction-and-distance attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the
HIP path and imports nothing from it.

Source: "Geometric direction-and-distance attention" (BioTorch exercise,
ESM3-style geometric attention), section "Required behavior". Per batch
element b, residue i, head h (frames T_i = (R_i, t_i), R_i maps local column
vectors to the global frame):

  qd_i = R_i q_direction_i            kd_j = R_j k_direction_j
  qp_i = R_i q_point_i + t_i          kp_j = R_j k_point_j + t_j
  a_ijh = ( softplus(direction_scale_h) (qd_i . kd_j)
            - softplus(distance_scale_h) ||qp_i - kp_j|| ) / sqrt(3)
          (the Euclidean distance itself, not its square, no epsilon)
  allowed_ijh = frame_mask_i and frame_mask_j and pair_mask[b, h, i, j]
  A_ijh = softmax over allowed j of a_ijh; rows with no allowed key are 0
  vectors_ihm = R_i^T sum_j A_ijh (R_j values_jhm)   (rotation only)
  output_i = flatten_{h, m, xyz}(vectors_i) @ output_weight + output_bias,
             forced to 0 when no head of query i has an allowed key.

Pinning status (tests/test_dirdist_pins.py): pinned against a scalar-loop
brute force, textbook attention through the library routine when the
distance term vanishes, hand-worked closed forms for the unsquared distance
and for the value transport convention, rigid-motion invariance, residue
permutation equivariance, the mask and readout rules, and softplus at
extreme logits.
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def softplus(x):
    """log(1 + exp(x)) without overflow: max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=F64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def dirdist_attention(rot, trans, q_direction, k_direction, q_point, k_point, values,
                      direction_scale, distance_scale, output_weight, output_bias=None,
                      frame_mask=None, pair_mask=None, rows=None):
    """Direction-and-distance attention in fp64 with explicit [N, N] tensors.

    ``rows`` (optional 1-D int array) restricts the queries to those residues
    (each query row is independent); the outputs then have N' = len(rows)
    along the query axis and every key.

    rot [B,N,3,3], trans [B,N,3]; q_direction, k_direction, q_point, k_point
    [B,N,H,3]; values [B,N,H,M,3]; direction_scale, distance_scale [H] (raw
    logits); output_weight [H*M*3, Cout]; output_bias [Cout] or None;
    frame_mask [B,N] (None: all valid); pair_mask broadcastable to [B,H,N,N]
    or None.

    Returns dict: "vectors" [B,N,H,M,3], "attention" [B,H,N,N],
    "output" [B,N,Cout], all float64.
    """
    rot, trans = np.asarray(rot, F64), np.asarray(trans, F64)
    qdir, kdir = np.asarray(q_direction, F64), np.asarray(k_direction, F64)
    qpt, kpt = np.asarray(q_point, F64), np.asarray(k_point, F64)
    val = np.asarray(values, F64)
    W = np.asarray(output_weight, F64)
    B, N, H, M, _ = val.shape
    Cout = W.shape[1]
    fm = np.ones((B, N), bool) if frame_mask is None else np.asarray(frame_mask).astype(bool)
    pm = np.ones((B, H, N, N), bool) if pair_mask is None else \
        np.broadcast_to(np.asarray(pair_mask).astype(bool), (B, H, N, N))
    cd = softplus(direction_scale) / math.sqrt(3.0)       # [H]
    cs = softplus(distance_scale) / math.sqrt(3.0)

    # directions rotate; points rotate and translate; values rotate only
    qd = np.einsum("bnxy,bnhy->bnhx", rot, qdir)
    kd = np.einsum("bnxy,bnhy->bnhx", rot, kdir)
    qp = np.einsum("bnxy,bnhy->bnhx", rot, qpt) + trans[:, :, None, :]
    kp = np.einsum("bnxy,bnhy->bnhx", rot, kpt) + trans[:, :, None, :]
    gv = np.einsum("bnxy,bnhmy->bnhmx", rot, val)

    qi = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    qd, qp, rot_q = qd[:, qi], qp[:, qi], rot[:, qi]
    pm = pm[:, :, qi]
    dots = np.einsum("bihx,bjhx->bhij", qd, kd)
    diff = qp.transpose(0, 2, 1, 3)[:, :, :, None, :] - kp.transpose(0, 2, 1, 3)[:, :, None, :, :]
    dist = np.sqrt(np.sum(diff * diff, axis=-1))                       # [B,H,N,N]
    logit = cd[None, :, None, None] * dots - cs[None, :, None, None] * dist

    allowed = fm[:, None, qi, None] & fm[:, None, None, :] & pm         # [B,H,N',N]
    lg = np.where(allowed, logit, -np.inf)
    m = lg.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(lg - m), 0.0)
    den = e.sum(axis=-1, keepdims=True)
    att = np.divide(e, den, out=np.zeros_like(e), where=den > 0)

    agg = np.einsum("bhij,bjhmx->bihmx", att, gv)                       # global frame
    vectors = np.einsum("biyx,bihmy->bihmx", rot_q, agg)                # R_i^T
    flat = vectors.reshape(B, len(qi), H * M * 3)
    out = flat @ W
    if output_bias is not None:
        out = out + np.asarray(output_bias, F64)[None, None, :]
    any_key = allowed.any(axis=-1).any(axis=1)                          # [B,N]
    out = np.where(any_key[:, :, None], out, 0.0)
    return {"vectors": vectors + 0.0, "attention": att + 0.0, "output": out + 0.0}
