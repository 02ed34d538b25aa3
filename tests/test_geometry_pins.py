"""Pins of the frame and distance-attention oracles (CPU only).

Frames ("Flash Invariant Point Attention", Figure 1: C-alpha is the centre,
C-alpha -> N and C-alpha -> C span the frame, completed by Gram-Schmidt):
  * orthonormal, right-handed rotations;
  * the atoms' local coordinates: C on the first axis, N in the plane of the
    first two axes on the positive side of the second;
  * SE(3) equivariance;
  * two hand-worked closed forms.
Distance attention (MEET section 2.2, eq. 6-8):
  * textbook softmax attention (library routine) when s = 0;
  * the pages' lifting identity: the logit equals rho <[q, -phi_s(x)], [k, psi_s(x)]>,
    computed through the library attention routine;
  * invariance under a rigid motion of the points;
  * a two-residue closed form;
  * mask rules;
  * agreement with the IPA oracle configured to the same logit.
Planted mistakes in copies of the oracles must be caught by these pins.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import geometry as geo
from oracle import ipa_forward
from workloads import MEET_WORKLOADS, make_backbone, make_meet_inputs

TINY = MEET_WORKLOADS["meet_tiny_fp32"].with_(L=20, H=3, C=8)


def _rand_rot(rng):
    u = rng.standard_normal(4)
    u /= np.linalg.norm(u)
    w, x, y, z = u
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
        [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
        [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)],
    ])


# ----------------------------------------------------------------------------
# frames from backbone atoms
# ----------------------------------------------------------------------------

def test_frames_orthonormal_right_handed():
    bb = make_backbone(2, 50, seed=1)
    rot, trans = geo.frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    eye = np.einsum("blxi,blxj->blij", rot, rot)
    assert np.abs(eye - np.eye(3)).max() < 1e-12
    assert np.abs(np.linalg.det(rot) - 1.0).max() < 1e-12
    assert np.array_equal(trans, bb["ca"].astype(np.float64))


def _check_local_coords(rot, bb):
    ca = bb["ca"].astype(np.float64)
    c_loc = np.einsum("blxi,blx->bli", rot, bb["c"] - ca)
    n_loc = np.einsum("blxi,blx->bli", rot, bb["n"] - ca)
    assert np.abs(c_loc[..., 1:]).max() < 1e-12
    assert np.abs(c_loc[..., 0] - np.linalg.norm(bb["c"] - ca, axis=-1)).max() < 1e-12
    assert np.abs(n_loc[..., 2]).max() < 1e-12
    assert n_loc[..., 1].min() > 0.0
    assert np.abs(np.linalg.norm(n_loc, axis=-1) - np.linalg.norm(bb["n"] - ca, axis=-1)).max() < 1e-12


def test_frames_local_atom_coordinates():
    bb = make_backbone(2, 64, seed=2)
    rot, _ = geo.frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    _check_local_coords(rot, bb)


@pytest.mark.parametrize("seed", [0, 3])
def test_frames_se3_equivariance(seed):
    rng = np.random.default_rng(seed)
    bb = {k: v.astype(np.float64) for k, v in make_backbone(1, 30, seed=seed).items()}
    Q = _rand_rot(rng)
    sft = rng.uniform(-50, 50, size=3)
    moved = {k: v @ Q.T + sft for k, v in bb.items()}
    r0, t0 = geo.frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    r1, t1 = geo.frames_from_atoms(moved["n"], moved["ca"], moved["c"])
    assert np.abs(r1 - np.einsum("xy,blyz->blxz", Q, r0)).max() < 1e-12
    assert np.abs(t1 - (t0 @ Q.T + sft)).max() < 1e-12


def test_frames_closed_forms():
    ca = np.array([[[1.0, 2.0, 3.0], [0.0, 0.0, 0.0]]])
    c = ca + np.array([[[2.0, 0.0, 0.0], [0.0, 0.0, 5.0]]])
    n = ca + np.array([[[1.0, 3.0, 0.0], [0.0, 4.0, 0.0]]])
    rot, trans = geo.frames_from_atoms(n, ca, c)
    assert np.abs(rot[0, 0] - np.eye(3)).max() < 1e-15
    # axes: e1 = z, e2 = y, e3 = z x y = -x; columns of R
    want = np.array([[0.0, 0.0, -1.0], [0.0, 1.0, 0.0], [1.0, 0.0, 0.0]])
    assert np.abs(rot[0, 1] - want).max() < 1e-15
    assert np.array_equal(trans, ca)


def test_planted_swapped_atoms_is_caught(monkeypatch):
    orig = geo.frames_from_atoms
    monkeypatch.setattr(geo, "frames_from_atoms", lambda n, ca, c: orig(c, ca, n))
    bb = make_backbone(1, 16, seed=4)
    rot, _ = geo.frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    with pytest.raises(AssertionError):
        _check_local_coords(rot, bb)


def test_planted_left_handed_frame_is_caught():
    bb = make_backbone(1, 16, seed=5)
    rot, _ = geo.frames_from_atoms(bb["n"], bb["ca"], bb["c"])
    bad = rot.copy()
    bad[..., 2] *= -1.0
    assert np.abs(np.linalg.det(bad) - 1.0).max() > 1.0


# ----------------------------------------------------------------------------
# distance-penalised attention
# ----------------------------------------------------------------------------

def _sdpa_heads(q, k, v, rho, bias=None):
    """Library attention per head, float64: q, k [L, H, d], v [L, H, e]."""
    outs = []
    for h in range(q.shape[1]):
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a[:, h][None])) for a in (q, k, v))
        m = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias[None]))
        outs.append(F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=float(rho[h]))[0].numpy())
    return np.stack(outs, axis=1)


def test_meet_textbook_reduction():
    inp = make_meet_inputs(TINY, seed=1)
    s0 = np.zeros_like(inp["s"])
    out = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], s0)
    q, k, v = (inp[n][0].astype(np.float64) for n in ("q", "k", "v"))
    ref = _sdpa_heads(q, k, v, inp["rho"])
    assert np.abs(out[0] - ref).max() < 1e-12


def _phi(x, s):
    cols = []
    for kk in range(3):
        cols += [x[:, kk] ** 2, np.ones(len(x)), -2.0 * x[:, kk]]
    return s * np.stack(cols, axis=-1)


def _psi(x, s):
    cols = []
    for kk in range(3):
        cols += [np.ones(len(x)), x[:, kk] ** 2, x[:, kk]]
    return s * np.stack(cols, axis=-1)


@pytest.mark.parametrize("seed", [0, 2])
def test_meet_lifting_identity_through_library_attention(seed):
    inp = make_meet_inputs(TINY, seed=seed)
    out = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"])
    x = inp["x"][0].astype(np.float64)
    q, k, v = (inp[n][0].astype(np.float64) for n in ("q", "k", "v"))
    H = q.shape[1]
    qa = np.stack([np.concatenate([q[:, h], -_phi(x, inp["s"][h])], axis=-1) for h in range(H)], axis=1)
    ka = np.stack([np.concatenate([k[:, h], _psi(x, inp["s"][h])], axis=-1) for h in range(H)], axis=1)
    ref = _sdpa_heads(qa, ka, v, inp["rho"])
    assert np.abs(out[0] - ref).max() < 1e-10


@pytest.mark.parametrize("seed", [0, 5])
def test_meet_rigid_invariance(seed):
    rng = np.random.default_rng(seed)
    inp = make_meet_inputs(TINY, seed=seed)
    Q = _rand_rot(rng)
    x2 = inp["x"].astype(np.float64) @ Q.T + rng.uniform(-100, 100, size=3)
    o1 = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"])
    o2 = geo.meet_attention(inp["q"], inp["k"], inp["v"], x2, inp["rho"], inp["s"])
    assert np.abs(o1 - o2).max() < 1e-10


@pytest.mark.parametrize("d", [0.5, 2.0, 4.0])
def test_meet_two_residue_closed_form(d):
    q = np.array([[[[0.3]], [[-0.7]]]])
    k = np.array([[[[1.1]], [[0.4]]]])
    v = np.array([[[[2.0]], [[-1.0]]]])
    x = np.array([[[0.0, 0.0, 0.0], [d, 0.0, 0.0]]])
    rho, s = np.array([0.8]), np.array([0.6])
    out = geo.meet_attention(q, k, v, x, rho, s)
    for i in range(2):
        l_self = rho[0] * q[0, i, 0, 0] * k[0, i, 0, 0]
        l_other = rho[0] * (q[0, i, 0, 0] * k[0, 1 - i, 0, 0] - s[0] ** 2 * d * d)
        a_self = 1.0 / (1.0 + math.exp(l_other - l_self))
        want = a_self * v[0, i, 0, 0] + (1.0 - a_self) * v[0, 1 - i, 0, 0]
        assert abs(out[0, i, 0, 0] - want) < 1e-14


def test_meet_mask_rules():
    w = TINY.with_(B=2, ragged=(8, 20))
    inp = make_meet_inputs(w, seed=3)
    out = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"], inp["mask"])
    for b in range(2):
        n = int(inp["lengths"][b])
        assert np.all(out[b, n:] == 0.0) and not np.signbit(out[b, n:]).any()
        sub = geo.meet_attention(inp["q"][b:b + 1, :n], inp["k"][b:b + 1, :n], inp["v"][b:b + 1, :n],
                                 inp["x"][b:b + 1, :n], inp["rho"], inp["s"])
        assert np.abs(out[b, :n] - sub[0]).max() < 1e-12
    allm = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"],
                              np.zeros_like(inp["mask"]))
    assert np.all(allm == 0.0) and not np.signbit(allm).any()


def test_meet_matches_ipa_configuration():
    """The IPA oracle with identity rotations, translations x, one zero local
    point per head, no pair term, w_L = 1, w_C = 2, gamma_h = rho_h s_h^2 and
    q scaled by rho_h sqrt(C) has the same logit, hence the same output."""
    inp = make_meet_inputs(TINY, seed=4)
    B, L, H, C = (inp["dims"][n] for n in ("B", "L", "H", "C"))
    out = geo.meet_attention(inp["q"], inp["k"], inp["v"], inp["x"], inp["rho"], inp["s"])
    ipa = dict(
        q=inp["q"].astype(np.float64) * (inp["rho"].astype(np.float64) * math.sqrt(C))[None, None, :, None],
        k=inp["k"], v=inp["v"],
        q_pts=np.zeros((B, L, H, 1, 3)), k_pts=np.zeros((B, L, H, 1, 3)), v_pts=np.zeros((B, L, H, 1, 3)),
        rot=np.broadcast_to(np.eye(3), (B, L, 3, 3)).copy(), trans=inp["x"],
        z1=np.zeros((B, L, 1, 8)), z2=np.zeros((B, L, 1, 8)), w_b=np.zeros((8, H)),
        gamma=inp["rho"].astype(np.float64) * inp["s"].astype(np.float64) ** 2,
        mask=None, w_L=1.0, w_C=2.0,
        dims=dict(B=B, L=L, H=H, C=C, Pqk=1, Pv=1, R=1, Cz=8),
    )
    ref = ipa_forward(ipa)["s"]
    assert np.abs(out - ref).max() < 1e-10


def _run_meet_pins():
    failures = 0
    for fn in (lambda: test_meet_lifting_identity_through_library_attention(0),
               lambda: test_meet_two_residue_closed_form(2.0),
               test_meet_mask_rules,
               test_meet_matches_ipa_configuration):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def _planted_meet(sign=-1.0, use_mask=True):
    """A copy of the distance-attention oracle with one mistake planted."""
    def meet(q, k, v, x, rho, s, mask=None):
        q, k, v, x = (np.asarray(a, dtype=np.float64) for a in (q, k, v, x))
        rho, s = np.asarray(rho, dtype=np.float64), np.asarray(s, dtype=np.float64)
        B, L, H, C = q.shape
        valid = np.ones((B, L), bool) if (mask is None or not use_mask) else np.asarray(mask).astype(bool)
        out = np.zeros((B, L, H, C))
        for b in range(B):
            d2 = np.sum((x[b][:, None] - x[b][None]) ** 2, axis=-1)
            lg = rho * (np.einsum("ihc,jhc->ijh", q[b], k[b]) + sign * (s * s) * d2[:, :, None])
            lg = np.where((valid[b][:, None] & valid[b][None, :])[:, :, None], lg, -np.inf)
            m = np.max(lg, axis=1, keepdims=True)
            p = np.exp(lg - np.where(np.isfinite(m), m, 0.0))
            den = p.sum(axis=1, keepdims=True)
            a = np.divide(p, den, out=np.zeros_like(p), where=den > 0)
            out[b] = np.einsum("ijh,jhc->ihc", a, v[b])
            out[b][~valid[b]] = 0.0
        return out + 0.0
    return meet


def test_planted_distance_sign_is_caught(monkeypatch):
    monkeypatch.setattr(geo, "meet_attention", _planted_meet(sign=+1.0))
    assert _run_meet_pins() > 0


def test_planted_ignored_mask_is_caught(monkeypatch):
    monkeypatch.setattr(geo, "meet_attention", _planted_meet(use_mask=False))
    assert _run_meet_pins() > 0


def test_unplanted_copy_passes(monkeypatch):
    monkeypatch.setattr(geo, "meet_attention", _planted_meet())
    assert _run_meet_pins() == 0
