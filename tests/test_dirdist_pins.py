"""Pins of the direction-and-distance attention oracle (CPU only).

"Geometric direction-and-distance attention", Required behavior:
  * a scalar-loop brute force written separately agrees on tiny inputs;
  * with both points at the origin of identity frames the distance term
    vanishes and the op is textbook softmax attention with scale
    softplus(direction_scale) / sqrt(3) (library routine);
  * hand-worked closed forms: the unsquared distance and its softplus scale,
    and the value transport R_i^T R_j v (no translation);
  * a rigid motion of every frame changes no output;
  * permuting residues permutes the outputs;
  * mask rules (frame validity, pair mask broadcasting, empty rows, the
    output forced to zero only when every head is empty) and the readout's
    H, M, xyz flattening order;
  * softplus at extreme logits.
Planted mistakes in copies of the oracle must be caught by these pins.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dirdist as dd
from oracle import dirdist_bruteforce
from workloads import DIRDIST_WORKLOADS, make_dirdist_inputs

TINY = DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(N=6, H=2, M=2, Cout=3, ragged=(4, 6))

ARGS = ("rot", "trans", "q_direction", "k_direction", "q_point", "k_point", "values",
        "direction_scale", "distance_scale", "output_weight", "output_bias",
        "frame_mask", "pair_mask")


def run(inp, **over):
    kw = {k: inp[k] for k in ARGS}
    kw.update(over)
    return dd.dirdist_attention(**kw)


def _rz(deg):
    c, s = math.cos(math.radians(deg)), math.sin(math.radians(deg))
    return np.array([[c, -s, 0], [s, c, 0], [0, 0, 1]])


def _rx(deg):
    c, s = math.cos(math.radians(deg)), math.sin(math.radians(deg))
    return np.array([[1, 0, 0], [0, c, -s], [0, s, c]])


def _rand_rot(rng):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def _blank(B, N, H, M, Cout=1):
    """Identity frames at the origin, zero features, all valid."""
    return dict(
        rot=np.broadcast_to(np.eye(3), (B, N, 3, 3)).copy(), trans=np.zeros((B, N, 3)),
        q_direction=np.zeros((B, N, H, 3)), k_direction=np.zeros((B, N, H, 3)),
        q_point=np.zeros((B, N, H, 3)), k_point=np.zeros((B, N, H, 3)),
        values=np.zeros((B, N, H, M, 3)), direction_scale=np.zeros(H), distance_scale=np.zeros(H),
        output_weight=np.zeros((H * M * 3, Cout)), output_bias=None,
        frame_mask=np.ones((B, N), np.uint8), pair_mask=None)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_scalar_bruteforce(seed):
    inp = make_dirdist_inputs(TINY, seed=seed)
    ref = dirdist_bruteforce(inp)
    got = run(inp)
    for k in ("vectors", "attention", "output"):
        assert np.abs(got[k] - ref[k]).max() < 1e-12, k


def test_bruteforce_broadcast_pair_mask():
    inp = make_dirdist_inputs(TINY.with_(pair_mask="shared"), seed=5)
    assert inp["pair_mask"].shape == (6, 6)
    ref = dirdist_bruteforce(inp)
    got = run(inp)
    for k in ("vectors", "attention", "output"):
        assert np.abs(got[k] - ref[k]).max() < 1e-12, k


@pytest.mark.parametrize("seed", [0, 1])
def test_textbook_attention_when_points_coincide(seed):
    """Identity frames, zero translations and zero points: every distance is
    zero, so the logit is softplus(a)/sqrt(3) qd.kd and the aggregated values
    are plain attention over the flattened (M, xyz) value channels."""
    rng = np.random.default_rng(seed)
    B, N, H, M = 2, 9, 3, 2
    inp = _blank(B, N, H, M)
    inp["q_direction"] = rng.standard_normal((B, N, H, 3))
    inp["k_direction"] = rng.standard_normal((B, N, H, 3))
    inp["values"] = rng.standard_normal((B, N, H, M, 3))
    inp["direction_scale"] = rng.standard_normal(H)
    inp["distance_scale"] = rng.standard_normal(H) + 3.0      # large, but the distance is 0
    got = run(inp)["vectors"]
    sc = torch.nn.functional.softplus(torch.tensor(inp["direction_scale"])) / math.sqrt(3.0)
    q = torch.tensor(inp["q_direction"]).permute(0, 2, 1, 3) * sc[None, :, None, None]
    k = torch.tensor(inp["k_direction"]).permute(0, 2, 1, 3)
    v = torch.tensor(inp["values"]).reshape(B, N, H, M * 3).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(q, k, v, scale=1.0)           # [B,H,N,3M]
    ref = ref.permute(0, 2, 1, 3).reshape(B, N, H, M, 3).numpy()
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("b_logit", [0.0, 1.3, -2.0])
def test_unsquared_distance_closed_form(b_logit):
    """One query at the origin, keys at distances 0 (itself), 1 and 4, no
    direction term: A = [1, e^-c, e^-4c] / Z with c = softplus(b) / sqrt(3)."""
    inp = _blank(1, 3, 1, 1)
    inp["trans"][0, 1] = [0.6, 0.8, 0.0]          # |.| = 1
    inp["trans"][0, 2] = [0.0, 0.0, -4.0]         # |.| = 4
    inp["distance_scale"] = np.array([b_logit])
    inp["values"][0, :, 0, 0, 0] = [1.0, 10.0, 100.0]
    c = math.log1p(math.exp(b_logit)) / math.sqrt(3.0)
    e = np.array([1.0, math.exp(-c), math.exp(-4.0 * c)])
    a = e / e.sum()
    got = run(inp)
    assert np.abs(got["attention"][0, 0, 0] - a).max() < 1e-14
    assert abs(got["vectors"][0, 0, 0, 0, 0] - (a[0] + 10 * a[1] + 100 * a[2])) < 1e-12


def test_value_transport_closed_form():
    """Query 0 with R_0 = Rz(90) may only see key 1 with R_1 = Rx(90): its
    vectors are R_0^T R_1 v, worked by hand, whatever the translations."""
    inp = _blank(1, 2, 1, 2)
    inp["rot"][0, 0] = _rz(90)
    inp["rot"][0, 1] = _rx(90)
    inp["trans"][0] = [[500.0, -3.0, 7.0], [-40.0, 20.0, 1.0]]
    inp["values"][0, 1, 0] = [[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]]
    inp["pair_mask"] = np.array([[0, 1], [1, 1]], np.uint8)
    got = run(inp)["vectors"][0, 0, 0]
    # Rx(90) e_x = e_x, Rz(-90) e_x = -e_y ; Rx(90) e_y = e_z, Rz(-90) e_z = e_z
    assert np.abs(got - np.array([[0.0, -1.0, 0.0], [0.0, 0.0, 1.0]])).max() < 1e-12


def test_direction_closed_form():
    """Two keys, no distance term: logits softplus(a)/sqrt(3) (R_i qd).(R_j kd)."""
    inp = _blank(1, 2, 1, 1)
    inp["rot"][0, 1] = _rz(90)
    inp["q_direction"][0, 0, 0] = [0.0, 2.0, 0.0]
    inp["k_direction"][0, 0, 0] = [0.0, 1.0, 0.0]    # global (0, 1, 0): dot 2
    inp["k_direction"][0, 1, 0] = [0.0, -1.0, 0.0]   # global Rz(90)(-e_y) = e_x: dot 0
    inp["direction_scale"] = np.array([0.5])
    cd = math.log1p(math.exp(0.5)) / math.sqrt(3.0)
    e = np.array([math.exp(2.0 * cd), 1.0])
    got = run(inp)["attention"][0, 0, 0]
    assert np.abs(got - e / e.sum()).max() < 1e-14


@pytest.mark.parametrize("seed", [0, 1])
def test_rigid_motion_invariance(seed):
    rng = np.random.default_rng(seed)
    inp = make_dirdist_inputs(TINY.with_(N=11, ragged=None), seed=seed)
    G = _rand_rot(rng)
    u = rng.standard_normal(3) * 50
    moved = dict(inp)
    moved["rot"] = np.einsum("xy,bnyz->bnxz", G, inp["rot"].astype(np.float64))
    moved["trans"] = np.einsum("xy,bny->bnx", G, inp["trans"].astype(np.float64)) + u
    a, b = run(inp), run(moved)
    for k in ("vectors", "attention", "output"):
        assert np.abs(a[k] - b[k]).max() < 1e-10, k


def test_permutation_equivariance():
    inp = make_dirdist_inputs(TINY.with_(N=7, ragged=None), seed=3)
    perm = np.random.default_rng(0).permutation(7)
    p = dict(inp)
    for k in ("rot", "trans", "q_direction", "k_direction", "q_point", "k_point", "values", "frame_mask"):
        p[k] = inp[k][:, perm]
    p["pair_mask"] = inp["pair_mask"][:, :, perm][:, :, :, perm]
    a, b = run(inp), run(p)
    assert np.abs(a["vectors"][:, perm] - b["vectors"]).max() < 1e-12
    assert np.abs(a["output"][:, perm] - b["output"]).max() < 1e-12
    assert np.abs(a["attention"][:, :, perm][:, :, :, perm] - b["attention"]).max() < 1e-12


def test_mask_rules():
    inp = make_dirdist_inputs(TINY.with_(N=6, H=2, ragged=None, pair_mask=None), seed=4)
    inp["frame_mask"] = np.array([[1, 1, 0, 1, 1, 1], [1, 1, 1, 1, 1, 1]], np.uint8)
    pm = np.ones((2, 2, 6, 6), np.uint8)
    pm[0, :, 3, :] = 0                 # query 3: no key in any head
    pm[0, 1, 4, :] = 0                 # query 4: no key in head 1 only
    out = run(inp, pair_mask=pm)
    # invalid frame: no output, no attention from or to it
    assert np.all(out["output"][0, 2] == 0) and np.all(out["vectors"][0, 2] == 0)
    assert np.all(out["attention"][0, :, 2, :] == 0) and np.all(out["attention"][0, :, :, 2] == 0)
    # every head empty: output zero despite the bias
    assert np.all(out["output"][0, 3] == 0) and np.all(out["vectors"][0, 3] == 0)
    # one head empty: its vectors are zero, the output is not
    assert np.all(out["vectors"][0, 4, 1] == 0) and np.all(out["attention"][0, 1, 4] == 0)
    assert np.abs(out["output"][0, 4]).max() > 0
    assert abs(out["attention"][0, 0, 4].sum() - 1.0) < 1e-12
    # rows sum to one over allowed keys, all outputs are positive zeros where zero
    s = out["attention"].sum(-1)
    assert np.all((np.abs(s - 1) < 1e-12) | (s == 0))
    for k in ("vectors", "attention", "output"):
        z = out[k] == 0
        assert not np.signbit(out[k][z]).any()


@pytest.mark.parametrize("shape", [(6, 6), (2, 1, 6, 6), (1, 2, 6, 6), (2, 2, 6, 6)])
def test_pair_mask_broadcasting(shape):
    inp = make_dirdist_inputs(TINY.with_(N=6, H=2, ragged=None, pair_mask=None), seed=6)
    pm = (np.random.default_rng(1).random(shape) < 0.7).astype(np.uint8)
    a = run(inp, pair_mask=pm)
    b = run(inp, pair_mask=np.broadcast_to(pm, (2, 2, 6, 6)).copy())
    for k in ("vectors", "attention", "output"):
        assert np.array_equal(a[k], b[k])


def test_readout_flatten_order():
    """A one-hot output weight at row (h M + m) 3 + x reads vectors[h, m, x]."""
    inp = make_dirdist_inputs(TINY.with_(N=5, H=2, M=3, Cout=4, ragged=None, pair_mask=None), seed=7)
    W = np.zeros((2 * 3 * 3, 4))
    picks = [(0, 0, 0), (1, 2, 1), (0, 1, 2), (1, 0, 2)]
    for c, (h, m, x) in enumerate(picks):
        W[(h * 3 + m) * 3 + x, c] = 1.0
    out = run(inp, output_weight=W, output_bias=np.arange(4.0))
    for c, (h, m, x) in enumerate(picks):
        assert np.abs(out["output"][..., c] - (out["vectors"][..., h, m, x] + c)).max() < 1e-12


def test_softplus_extremes():
    assert dd.softplus(1000.0) == 1000.0
    assert 0 < dd.softplus(-745.0) < 1e-300
    assert abs(dd.softplus(0.0) - math.log(2.0)) < 1e-16
    inp = make_dirdist_inputs(TINY.with_(ragged=None), seed=8)
    out = run(inp, direction_scale=np.array([800.0, -800.0]), distance_scale=np.array([-900.0, 30.0]))
    for k in ("vectors", "attention", "output"):
        assert np.isfinite(out[k]).all()


def test_zero_displacement_is_finite():
    inp = _blank(1, 2, 1, 1)
    inp["values"][0, :, 0, 0] = [[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]]
    out = run(inp)
    assert np.abs(out["attention"][0, 0] - 0.5).max() < 1e-15
    assert np.abs(out["vectors"][0, 0, 0, 0] - [2.5, 3.5, 4.5]).max() < 1e-15


# ---------------------------------------------------------------------------
# planted mistakes: each copy of the oracle carries one, and a pin catches it
# ---------------------------------------------------------------------------
def _planted(squared=False, no_sqrt3=False, transpose_back=False, translate_values=False,
             keep_bias=False, plain_scales=False):
    def f(rot, trans, q_direction, k_direction, q_point, k_point, values, direction_scale,
          distance_scale, output_weight, output_bias=None, frame_mask=None, pair_mask=None):
        rot, trans = np.asarray(rot, float), np.asarray(trans, float)
        val = np.asarray(values, float)
        B, N, H, M, _ = val.shape
        fm = np.ones((B, N), bool) if frame_mask is None else np.asarray(frame_mask).astype(bool)
        pm = np.ones((B, H, N, N), bool) if pair_mask is None else \
            np.broadcast_to(np.asarray(pair_mask).astype(bool), (B, H, N, N))
        sp = (lambda x: np.asarray(x, float)) if plain_scales else dd.softplus
        k3 = 1.0 if no_sqrt3 else math.sqrt(3.0)
        cd, cs = sp(direction_scale) / k3, sp(distance_scale) / k3
        qd = np.einsum("bnxy,bnhy->bnhx", rot, q_direction)
        kd = np.einsum("bnxy,bnhy->bnhx", rot, k_direction)
        qp = np.einsum("bnxy,bnhy->bnhx", rot, q_point) + trans[:, :, None]
        kp = np.einsum("bnxy,bnhy->bnhx", rot, k_point) + trans[:, :, None]
        gv = np.einsum("bnxy,bnhmy->bnhmx", rot, val)
        if translate_values:
            gv = gv + trans[:, :, None, None, :]
        diff = qp.transpose(0, 2, 1, 3)[:, :, :, None] - kp.transpose(0, 2, 1, 3)[:, :, None]
        d2 = np.sum(diff * diff, -1)
        dist = d2 if squared else np.sqrt(d2)
        lg = cd[None, :, None, None] * np.einsum("bihx,bjhx->bhij", qd, kd) - cs[None, :, None, None] * dist
        allowed = fm[:, None, :, None] & fm[:, None, None, :] & pm
        lg = np.where(allowed, lg, -np.inf)
        m = lg.max(-1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(allowed, np.exp(lg - m), 0.0)
        den = e.sum(-1, keepdims=True)
        att = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
        agg = np.einsum("bhij,bjhmx->bihmx", att, gv)
        eq = "bixy,bihmy->bihmx" if transpose_back else "biyx,bihmy->bihmx"
        vec = np.einsum(eq, rot, agg)
        out = vec.reshape(B, N, -1) @ np.asarray(output_weight, float)
        if output_bias is not None:
            out = out + np.asarray(output_bias, float)
        if not keep_bias:
            out = np.where(allowed.any(-1).any(1)[:, :, None], out, 0.0)
        return {"vectors": vec, "attention": att, "output": out}
    return f


PINS = [test_unsquared_distance_closed_form, test_value_transport_closed_form,
        test_direction_closed_form, test_rigid_motion_invariance, test_mask_rules,
        test_textbook_attention_when_points_coincide, test_softplus_extremes]


def _caught(monkeypatch, **mistake):
    monkeypatch.setattr(dd, "dirdist_attention", _planted(**mistake))
    failed = 0
    for t in PINS:
        params = {test_unsquared_distance_closed_form: {"b_logit": 1.3},
                  test_rigid_motion_invariance: {"seed": 0},
                  test_textbook_attention_when_points_coincide: {"seed": 0}}.get(t, {})
        try:
            with np.errstate(all="ignore"):
                t(**params)
        except (AssertionError, FloatingPointError):
            failed += 1
    return failed


@pytest.mark.parametrize("mistake", ["squared", "no_sqrt3", "transpose_back", "translate_values",
                                     "keep_bias", "plain_scales"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    assert _caught(monkeypatch, **{mistake: True}) > 0


def test_unplanted_copy_passes(monkeypatch):
    assert _caught(monkeypatch) == 0


def test_row_subset_matches_full():
    inp = make_dirdist_inputs(TINY.with_(N=9, ragged=(6, 9), pair_mask="full"), seed=9)
    full = run(inp)
    rows = np.array([0, 3, 4, 8])
    sub = dd.dirdist_attention(**{k: inp[k] for k in ARGS}, rows=rows)
    assert np.array_equal(sub["vectors"], full["vectors"][:, rows])
    assert np.array_equal(sub["attention"], full["attention"][:, :, rows])
    assert np.abs(sub["output"] - full["output"][:, rows]).max() < 1e-14
