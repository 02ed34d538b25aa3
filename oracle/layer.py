"""fp64 CPU oracle for the full IPA layer around the attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``. It shares no code with the
HIP path and imports nothing from it.

The layer, as read here (the pages fix the attention, not its wrap):
"Flash Invariant Point Attention", TL;DR and abstract: per-residue scalar,
point and factorised pair features (z_ij = z1_i * z2_j) feed the attention.
They are produced from the single representation s by one affine map,
  x = s W_in + b_in,  x = [q | k | v | q_pts | k_pts | v_pts | z1 | z2]
(each block flattened head-major, points as (head, point, xyz), pair
factors as (rank, channel)), the attention runs (``ipa_forward``), and its
four outputs are read out by a second affine map over their concatenation,
  y = [o_s | o_pts | o_norm | o_pair] W_out + b_out
flattened head-major with xyz last, the order the readout of "Geometric
direction-and-distance attention" (Required behavior) fixes for its own
vectors. Rows whose mask entry is 0 give y = +0.0 (the bias does not revive
an empty row, as on that page). For storage "bf16" the projected features
are rounded to bfloat16 (nearest even) before the attention, as the
kernels store them.

Pinning status (tests/test_layer_pins.py): with selection weights the layer
reduces to ``ipa_forward`` (itself pinned) plus a known readout; the
concatenation order is checked with one-hot readout weights; the affine
maps against a scalar loop; the row-restricted form against the full one.
"""

from __future__ import annotations

import numpy as np
import torch

from .ipa_oracle import ipa_forward

F64 = np.float64


def split_sizes(d: dict) -> list[tuple[str, tuple]]:
    """Column blocks of x = s W_in + b_in, in order, with their shapes per row."""
    H, C, P, Pv, R, Cz = (d[n] for n in ("H", "C", "Pqk", "Pv", "R", "Cz"))
    return [("q", (H, C)), ("k", (H, C)), ("v", (H, C)), ("q_pts", (H, P, 3)), ("k_pts", (H, P, 3)),
            ("v_pts", (H, Pv, 3)), ("z1", (R, Cz)), ("z2", (R, Cz))]


def in_width(d: dict) -> int:
    return sum(int(np.prod(shp)) for _, shp in split_sizes(d))


def out_width(d: dict) -> int:
    return d["H"] * (d["C"] + 3 * d["Pv"] + d["Pv"] + d["Cz"])


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def ipa_layer(inp: dict, rows=None) -> np.ndarray:
    """The layer in fp64 (bf16-rounded features for bf16 storage).

    inp: "s" [B,L,c_s], "rot", "trans", "mask", "w_in" [c_s, Nin],
    "b_in" [Nin], "w_b", "gamma", "w_L", "w_C", "w_out" [Nout, c_s],
    "b_out" [c_s], "dims", "dtype". Returns y [B,L,c_s] float64, or
    [B,L',c_s] for the query rows ``rows`` only (each output row depends on
    every residue's features but on its own attention row alone).
    """
    d = inp["dims"]
    B, L = d["B"], d["L"]
    s = np.asarray(inp["s"], F64)
    x = s @ np.asarray(inp["w_in"], F64) + np.asarray(inp["b_in"], F64)
    feats, c0 = {}, 0
    for name, shp in split_sizes(d):
        n = int(np.prod(shp))
        f = x[:, :, c0:c0 + n].reshape((B, L) + shp)
        feats[name] = _bf16(f) if inp["dtype"] == "bf16" else f
        c0 += n
    fwd_in = dict(feats)
    fwd_in.update(rot=inp["rot"], trans=inp["trans"], w_b=inp["w_b"], gamma=inp["gamma"],
                  mask=inp["mask"], w_L=inp["w_L"], w_C=inp["w_C"], dims=d)
    sel = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    o = ipa_forward(fwd_in, rows=None if rows is None else sel)
    n = len(sel)
    cat = np.concatenate([o["s"].reshape(B, n, -1), o["pts"].reshape(B, n, -1),
                          o["pts_norm"].reshape(B, n, -1), o["pair"].reshape(B, n, -1)], axis=-1)
    y = cat @ np.asarray(inp["w_out"], F64) + np.asarray(inp["b_out"], F64)
    keep = np.asarray(inp["mask"]).astype(bool)[:, sel]
    return np.where(keep[..., None], y, 0.0) + 0.0
