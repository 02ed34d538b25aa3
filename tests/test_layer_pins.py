"""Pins of the IPA layer oracle (CPU only).

  * with selection weights (W_in copies given features out of s, b_in = 0)
    the layer's attention inputs are exactly those features, so the layer
    equals ipa_forward (pinned elsewhere) followed by the readout;
  * one-hot readout rows pick o_s, o_pts, o_norm, o_pair in the documented
    flattened order (head-major, xyz last);
  * the two affine maps agree with a scalar loop on a tiny case;
  * masked rows give +0.0 despite the readout bias.
"""

import numpy as np

from oracle import ipa_forward
from oracle.layer import in_width, ipa_layer, out_width, split_sizes
from workloads import WORKLOADS, make_inputs, make_layer_inputs

TINY = WORKLOADS["tiny_fp32"].with_(L=6, H=2, C=3, Pqk=2, Pv=2, R=2, Cz=4)


def _selection_inputs(seed=0):
    """s holds the features of make_inputs(TINY) side by side; W_in = I."""
    base = make_inputs(TINY, seed=seed)
    d = TINY.dims()
    B, L = d["B"], d["L"]
    cols = [base[n].astype(np.float64).reshape(B, L, -1) for n, _ in split_sizes(d)]
    s = np.concatenate(cols, axis=-1)
    n_in = in_width(d)
    assert s.shape[-1] == n_in
    rng = np.random.default_rng(seed)
    n_out = out_width(d)
    inp = dict(s=s, rot=base["rot"], trans=base["trans"], mask=base["mask"], w_in=np.eye(n_in),
               b_in=np.zeros(n_in), w_b=base["w_b"], gamma=base["gamma"], w_L=base["w_L"],
               w_C=base["w_C"], w_out=rng.standard_normal((n_out, 5)), b_out=rng.standard_normal(5),
               dims=d, dtype="fp32")
    return base, inp


def test_selection_weights_reduce_to_the_attention():
    base, inp = _selection_inputs(1)
    y = ipa_layer(inp)
    o = ipa_forward(base)
    B, L = 1, TINY.L
    cat = np.concatenate([o["s"].reshape(B, L, -1), o["pts"].reshape(B, L, -1),
                          o["pts_norm"].reshape(B, L, -1), o["pair"].reshape(B, L, -1)], axis=-1)
    assert np.abs(y - (cat @ inp["w_out"] + inp["b_out"])).max() < 1e-12


def test_readout_order():
    base, inp = _selection_inputs(2)
    d = TINY.dims()
    H, C, Pv, Cz = d["H"], d["C"], d["Pv"], d["Cz"]
    o = ipa_forward(base)
    n_out = out_width(d)
    picks = {"s(1,2)": (1 * C + 2, o["s"][0, :, 1, 2]),
             "pts(1,0,z)": (H * C + (1 * Pv + 0) * 3 + 2, o["pts"][0, :, 1, 0, 2]),
             "norm(0,1)": (H * C + 3 * H * Pv + 0 * Pv + 1, o["pts_norm"][0, :, 0, 1]),
             "pair(1,3)": (H * C + 4 * H * Pv + 1 * Cz + 3, o["pair"][0, :, 1, 3])}
    W = np.zeros((n_out, len(picks)))
    for c, (row, _) in enumerate(picks.values()):
        W[row, c] = 1.0
    inp["w_out"], inp["b_out"] = W, np.zeros(len(picks))
    y = ipa_layer(inp)
    for c, (name, (_, ref)) in enumerate(picks.items()):
        assert np.abs(y[0, :, c] - ref).max() < 1e-12, name


def test_affine_maps_against_a_loop():
    inp = make_layer_inputs(TINY, c_s=5, seed=3)
    s, W, b = inp["s"].astype(np.float64), inp["w_in"].astype(np.float64), inp["b_in"].astype(np.float64)
    x = np.zeros((1, TINY.L, W.shape[1]))
    for i in range(TINY.L):
        for n in range(W.shape[1]):
            acc = b[n]
            for k in range(5):
                acc += s[0, i, k] * W[k, n]
            x[0, i, n] = acc
    # the layer with identity readout over its own projections equals the
    # attention on the loop-projected features
    d = TINY.dims()
    feats, c0 = {}, 0
    for name, shp in split_sizes(d):
        n = int(np.prod(shp))
        feats[name] = x[:, :, c0:c0 + n].reshape((1, TINY.L) + shp)
        c0 += n
    fwd = dict(feats, rot=inp["rot"], trans=inp["trans"], w_b=inp["w_b"], gamma=inp["gamma"],
               mask=inp["mask"], w_L=inp["w_L"], w_C=inp["w_C"], dims=d)
    o = ipa_forward(fwd)
    cat = np.concatenate([o["s"].reshape(1, TINY.L, -1), o["pts"].reshape(1, TINY.L, -1),
                          o["pts_norm"].reshape(1, TINY.L, -1), o["pair"].reshape(1, TINY.L, -1)], -1)
    ref = cat @ inp["w_out"].astype(np.float64) + inp["b_out"]
    assert np.abs(ipa_layer(inp) - ref).max() < 1e-10


def test_masked_rows_are_zero():
    w = WORKLOADS["ragged_batch"].with_(B=2, L=10, H=2, C=3, Pqk=2, Pv=2, R=1, Cz=4, ragged=(5, 10),
                                        dtype="fp32")
    inp = make_layer_inputs(w, c_s=7, seed=4)
    y = ipa_layer(inp)
    pad = inp["mask"] == 0
    assert pad.any() and np.all(y[pad] == 0) and not np.signbit(y[pad]).any()
    assert np.abs(y[~pad]).max() > 0


def test_row_restricted_layer_matches_full():
    w = WORKLOADS["ragged_batch"].with_(B=2, L=12, H=2, C=3, Pqk=2, Pv=2, R=1, Cz=4, ragged=(6, 12),
                                        dtype="bf16")
    inp = make_layer_inputs(w, c_s=6, seed=8)
    rows = np.array([0, 5, 11])
    full = ipa_layer(inp)
    part = ipa_layer(inp, rows=rows)
    assert part.shape == (2, 3, 6)
    assert np.abs(part - full[:, rows]).max() < 1e-12
