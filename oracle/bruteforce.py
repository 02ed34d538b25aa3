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
