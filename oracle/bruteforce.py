"""Scalar-loop IPA forward for tiny inputs (L <= 8).

TEST INFRASTRUCTURE ONLY (see ``oracle/ipa_oracle.py``). Plain Python loops
with ``math`` over (b, h, i, j, p, x): no numpy contraction, no broadcasting,
so an index or transpose slip in the vectorised oracle shows up as a
disagreement. It follows the same definition as ``ipa_oracle.ipa_forward``
("Flash Invariant Point Attention", TL;DR; MEET section 2.2 eq. 6;
"Geometric direction-and-distance attention", Required behavior).
"""

from __future__ import annotations

import math


def _g(R, t, x):
    # R x + t for one 3-vector
    return [R[a][0] * x[0] + R[a][1] * x[1] + R[a][2] * x[2] + t[a] for a in range(3)]


def ipa_bruteforce(inp: dict) -> dict:
    d = inp["dims"]
    B, L, H, C, Pqk, Pv, Rk, Cz = (d[n] for n in ("B", "L", "H", "C", "Pqk", "Pv", "R", "Cz"))
    tl = lambda name: inp[name].astype(float).tolist()
    q, k, v = tl("q"), tl("k"), tl("v")
    qp, kp, vp = tl("q_pts"), tl("k_pts"), tl("v_pts")
    rot, trans = tl("rot"), tl("trans")
    z1, z2 = tl("z1"), tl("z2")
    wb, gamma = tl("w_b"), tl("gamma")
    mask = inp["mask"].astype(int).tolist() if inp.get("mask") is not None else [[1] * L] * B
    wL, wC = float(inp["w_L"]), float(inp["w_C"])

    o_s = [[[[0.0] * C for _ in range(H)] for _ in range(L)] for _ in range(B)]
    o_p = [[[[[0.0] * 3 for _ in range(Pv)] for _ in range(H)] for _ in range(L)] for _ in range(B)]
    o_n = [[[[0.0] * Pv for _ in range(H)] for _ in range(L)] for _ in range(B)]
    o_z = [[[[0.0] * Cz for _ in range(H)] for _ in range(L)] for _ in range(B)]

    for b in range(B):
        Rb, tb = rot[b], trans[b]
        for h in range(H):
            for i in range(L):
                if not mask[b][i]:
                    continue
                logits = {}
                for j in range(L):
                    if not mask[b][j]:
                        continue
                    s = 0.0
                    for c in range(C):
                        s += q[b][i][h][c] * k[b][j][h][c]
                    s /= math.sqrt(C)
                    bias = 0.0
                    for c in range(Cz):
                        zij = 0.0
                        for r in range(Rk):
                            zij += z1[b][i][r][c] * z2[b][j][r][c]
                        bias += zij * wb[c][h]
                    dist = 0.0
                    for p in range(Pqk):
                        a = _g(Rb[i], tb[i], qp[b][i][h][p])
                        bb = _g(Rb[j], tb[j], kp[b][j][h][p])
                        for x in range(3):
                            dist += (a[x] - bb[x]) ** 2
                    logits[j] = wL * (s + bias - gamma[h] * wC / 2.0 * dist)
                mx = max(logits.values())
                ex = {j: math.exp(val - mx) for j, val in logits.items()}
                den = sum(ex.values())
                att = {j: e / den for j, e in ex.items()}
                og = [[0.0] * 3 for _ in range(Pv)]
                for j, a in att.items():
                    for c in range(C):
                        o_s[b][i][h][c] += a * v[b][j][h][c]
                    for p in range(Pv):
                        g = _g(Rb[j], tb[j], vp[b][j][h][p])
                        for x in range(3):
                            og[p][x] += a * g[x]
                    for c in range(Cz):
                        zij = 0.0
                        for r in range(Rk):
                            zij += z1[b][i][r][c] * z2[b][j][r][c]
                        o_z[b][i][h][c] += a * zij
                for p in range(Pv):
                    rel = [og[p][x] - tb[i][x] for x in range(3)]
                    loc = [sum(Rb[i][y][x] * rel[y] for y in range(3)) for x in range(3)]
                    o_p[b][i][h][p] = loc
                    o_n[b][i][h][p] = math.sqrt(sum(u * u for u in loc))
    import numpy as np
    return {"s": np.array(o_s), "pts": np.array(o_p), "pts_norm": np.array(o_n),
            "pair": np.array(o_z)}


def _softplus_scalar(x):
    # log(1 + e^x) evaluated without overflow for either sign of x
    return x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))


def dirdist_bruteforce(inp: dict) -> dict:
    """Scalar-loop direction-and-distance attention for tiny inputs (N <= 8).

    Follows "Geometric direction-and-distance attention", Required behavior,
    with plain loops over (b, h, i, j, m, x) and ``math`` only; the pair mask
    is read at its full [B, H, N, N] shape.
    """
    import numpy as np
    B, N, H, M, _ = inp["values"].shape
    tl = lambda name: np.asarray(inp[name], dtype=float).tolist()
    rot, trans = tl("rot"), tl("trans")
    qdir, kdir, qpt, kpt = tl("q_direction"), tl("k_direction"), tl("q_point"), tl("k_point")
    val = tl("values")
    W = tl("output_weight")
    Cout = len(W[0])
    bias = tl("output_bias") if inp.get("output_bias") is not None else [0.0] * Cout
    fm = np.asarray(inp["frame_mask"]).astype(int).tolist()
    pm_in = inp.get("pair_mask")
    pm = (np.broadcast_to(np.asarray(pm_in).astype(int), (B, H, N, N)).tolist()
          if pm_in is not None else [[[[1] * N for _ in range(N)] for _ in range(H)] for _ in range(B)])
    dsc, ssc = tl("direction_scale"), tl("distance_scale")

    def rotate(R, x):
        return [R[a][0] * x[0] + R[a][1] * x[1] + R[a][2] * x[2] for a in range(3)]

    vectors = [[[[[0.0] * 3 for _ in range(M)] for _ in range(H)] for _ in range(N)] for _ in range(B)]
    att = [[[[0.0] * N for _ in range(N)] for _ in range(H)] for _ in range(B)]
    output = [[[0.0] * Cout for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for i in range(N):
            any_head = False
            for h in range(H):
                cd = _softplus_scalar(dsc[h]) / math.sqrt(3.0)
                cs = _softplus_scalar(ssc[h]) / math.sqrt(3.0)
                qd = rotate(rot[b][i], qdir[b][i][h])
                qp = [u + t for u, t in zip(rotate(rot[b][i], qpt[b][i][h]), trans[b][i])]
                logits = {}
                for j in range(N):
                    if not (fm[b][i] and fm[b][j] and pm[b][h][i][j]):
                        continue
                    kd = rotate(rot[b][j], kdir[b][j][h])
                    kp = [u + t for u, t in zip(rotate(rot[b][j], kpt[b][j][h]), trans[b][j])]
                    dot = qd[0] * kd[0] + qd[1] * kd[1] + qd[2] * kd[2]
                    dist = math.sqrt(sum((qp[x] - kp[x]) ** 2 for x in range(3)))
                    logits[j] = cd * dot - cs * dist
                if not logits:
                    continue
                any_head = True
                mx = max(logits.values())
                den = sum(math.exp(a - mx) for a in logits.values())
                for j, a in logits.items():
                    att[b][h][i][j] = math.exp(a - mx) / den
                for m in range(M):
                    g = [0.0, 0.0, 0.0]
                    for j in logits:
                        gj = rotate(rot[b][j], val[b][j][h][m])
                        for x in range(3):
                            g[x] += att[b][h][i][j] * gj[x]
                    Ri = rot[b][i]
                    vectors[b][i][h][m] = [sum(Ri[y][x] * g[y] for y in range(3)) for x in range(3)]
            if any_head:
                for c in range(Cout):
                    acc = bias[c]
                    for h in range(H):
                        for m in range(M):
                            for x in range(3):
                                acc += vectors[b][i][h][m][x] * W[(h * M + m) * 3 + x][c]
                    output[b][i][c] = acc
    return {"vectors": np.array(vectors), "attention": np.array(att), "output": np.array(output)}
