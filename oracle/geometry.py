"""fp64 CPU oracle for two companions of the IPA forward: residue frames
from backbone atoms, and distance-penalised attention over one point per
residue.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the
HIP path and imports nothing from it.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def frames_from_atoms(n, ca, c):
    """Residue frames T = (R, t) from backbone atoms, in fp64.

    "Flash Invariant Point Attention", Figure 1: the C-alpha atom is the
    frame's centre, and the vectors from C-alpha to N and from C-alpha to C
    span the frame, completed by Gram-Schmidt. Reading taken here (the
    figure fixes neither the order nor the handedness): the first axis
    points from C-alpha to C, the second is the component of (N - C-alpha)
    orthogonal to it, the third is their cross product (right-handed), and
    the columns of R are these axes, so R maps local column vectors to the
    global frame (x_g = R x_l + t) with t = C-alpha.

    n, ca, c: [..., 3]. Returns rot [..., 3, 3], trans [..., 3].
    """
    n, ca, c = (np.asarray(a, dtype=F64) for a in (n, ca, c))
    v1 = c - ca
    v2 = n - ca
    e1 = v1 / np.linalg.norm(v1, axis=-1, keepdims=True)
    u2 = v2 - np.sum(e1 * v2, axis=-1, keepdims=True) * e1
    e2 = u2 / np.linalg.norm(u2, axis=-1, keepdims=True)
    e3 = np.cross(e1, e2)
    rot = np.stack([e1, e2, e3], axis=-1)
    return rot, ca.copy()


def meet_attention(q, k, v, x, rho, s, mask=None):
    """Attention whose logit carries an invariant squared-distance penalty,
    in fp64, with explicit O(L^2) tensors.

    "Scalable peptide design with memory-efficient equivariant transformers"
    (MEET), section 2.2, eq. 6: the logit of head h for query i and key j is
    rho_h (q_ih . k_jh - s_h^2 ||x_i - x_j||^2), with x_i one point per
    residue in the global frame. The softmax over keys and the weighted sum
    of the values follow the same section; masking follows the IPA
    convention used throughout (a key is allowed when both residues are
    valid, rows with no allowed key and invalid rows give +0.0).

    q, k, v: [B, L, H, C]; x: [B, L, 3]; rho, s: [H]; mask: [B, L] or None.
    Returns out [B, L, H, C].
    """
    q, k, v, x = (np.asarray(a, dtype=F64) for a in (q, k, v, x))
    rho = np.asarray(rho, dtype=F64)
    s = np.asarray(s, dtype=F64)
    B, L, H, C = q.shape
    valid = np.ones((B, L), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    out = np.zeros((B, L, H, C), dtype=F64)
    for b in range(B):
        diff = x[b][:, None, :] - x[b][None, :, :]
        d2 = np.sum(diff * diff, axis=-1)                                   # [L, L]
        dots = np.einsum("ihc,jhc->ijh", q[b], k[b])                        # [L, L, H]
        logit = rho[None, None, :] * (dots - (s * s)[None, None, :] * d2[:, :, None])
        allowed = valid[b][:, None] & valid[b][None, :]
        for h in range(H):
            lg = np.where(allowed, logit[:, :, h], -np.inf)
            m = np.max(lg, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            p = np.where(allowed, np.exp(lg - m), 0.0)
            den = np.sum(p, axis=1, keepdims=True)
            a = np.divide(p, den, out=np.zeros_like(p), where=den > 0)
            out[b, :, h, :] = a @ v[b][:, h, :]
        out[b][~valid[b]] = 0.0
    return out + 0.0
