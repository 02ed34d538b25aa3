"""Pins of the fp64 oracle to facts other than its own formula (CPU only).

Each test holds the oracle to something the pages or the mathematics fix:
  * textbook softmax attention (Bio2Token eq. 1, y = softmax(Q K^T) x) through
    the library routine torch.nn.functional.scaled_dot_product_attention;
  * the MEET lifting identity (section 2.2, eq. 7-8: concatenating -phi to the
    query and psi to the key reproduces the squared-distance logit), again
    through the library attention routine;
  * SE(3) invariance ("Flash Invariant Point Attention", TL;DR/abstract);
  * closed forms on degenerate inputs (one residue, two residues at a known
    distance, uniform attention);
  * permutation equivariance and the mask rules of "Geometric
    direction-and-distance attention" (allowed edge = both frames valid,
    all-masked rows give exact zeros, padding never influences valid rows).
A final group plants typical mistakes into a copy of the oracle and checks
that at least one pin catches each of them.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ipa_bruteforce, ipa_forward, ipa_lifted, to_global
from oracle import ipa_oracle as oracle_mod
from workloads import WORKLOADS, make_inputs, round_to_bf16

TINY = WORKLOADS["tiny_fp32"].with_(L=24, H=3, C=8, Cz=16)


def _inp(w=TINY, seed=0, **over):
    inp = make_inputs(w, seed=seed)
    for k, v in over.items():
        inp[k] = v
    return inp


def _rand_rot(rng):
    u = rng.standard_normal(4)
    u /= np.linalg.norm(u)
    w, x, y, z = u
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
        [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
        [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)],
    ])


def _sdpa(q, k, v, scale=1.0, bias=None):
    """Library attention on float64 CPU tensors: q [H,L,d], k [H,L,d], v [H,L,e]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    mask = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias))
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale).numpy()


# ----------------------------------------------------------------------------
# library-routine reductions
# ----------------------------------------------------------------------------

def test_textbook_attention_reduction():
    """gamma = 0 and W_b = 0 leave plain scaled softmax attention per head."""
    inp = _inp(seed=3)
    H = inp["dims"]["H"]
    inp["gamma"] = np.zeros(H, np.float32)
    inp["w_b"] = np.zeros_like(inp["w_b"])
    out = ipa_forward(inp)
    q = inp["q"][0].astype(np.float64).transpose(1, 0, 2)   # [H,L,C]
    k = inp["k"][0].astype(np.float64).transpose(1, 0, 2)
    v = inp["v"][0].astype(np.float64).transpose(1, 0, 2)
    C = q.shape[-1]
    ref = _sdpa(q, k, v, scale=inp["w_L"] / math.sqrt(C))   # [H,L,C]
    np.testing.assert_allclose(out["s"][0], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)
    # factorised pair output: sum_r z1_ir * softmax-average of z2_jr
    z1 = inp["z1"][0].astype(np.float64)
    z2 = inp["z2"][0].astype(np.float64)
    R = z1.shape[1]
    pair = 0
    for r in range(R):
        vz = np.broadcast_to(z2[None, :, r, :], (H,) + z2[:, r, :].shape)
        pair = pair + z1[None, :, r, :] * _sdpa(q, k, vz, scale=inp["w_L"] / math.sqrt(C))
    np.testing.assert_allclose(out["pair"][0], pair.transpose(1, 0, 2), rtol=0, atol=1e-12)


def _meet_phi(x, s):
    """MEET eq. 7: phi_s(x) = s (+)_k [x_k^2, 1, -2 x_k]; x [..., 3]."""
    cols = []
    for kk in range(3):
        cols += [x[..., kk] ** 2, np.ones_like(x[..., kk]), -2.0 * x[..., kk]]
    return s * np.stack(cols, axis=-1)


def _meet_psi(x, s):
    """MEET eq. 7: psi_s(x) = s (+)_k [1, x_k^2, x_k]; x [..., 3]."""
    cols = []
    for kk in range(3):
        cols += [np.ones_like(x[..., kk]), x[..., kk] ** 2, x[..., kk]]
    return s * np.stack(cols, axis=-1)


@pytest.mark.parametrize("seed", [0, 1])
def test_meet_lifting_identity_through_library_attention(seed):
    """Concatenate -phi to the query and psi to the key (MEET eq. 8), add the
    factorised pair bias as query/key columns, and run library attention:
    scalar, point and pair outputs equal the explicit-distance oracle."""
    inp = _inp(seed=seed)
    d = inp["dims"]
    H, C, Pqk, Pv, R, Cz = d["H"], d["C"], d["Pqk"], d["Pv"], d["R"], d["Cz"]
    out = ipa_forward(inp)
    rot = inp["rot"][0].astype(np.float64)
    trans = inp["trans"][0].astype(np.float64)
    Qg = to_global(rot, trans, inp["q_pts"][0].astype(np.float64))   # [L,H,P,3]
    Kg = to_global(rot, trans, inp["k_pts"][0].astype(np.float64))
    Vg = to_global(rot, trans, inp["v_pts"][0].astype(np.float64))
    L = Qg.shape[0]
    wL, wC = inp["w_L"], inp["w_C"]
    z1 = inp["z1"][0].astype(np.float64)
    z2 = inp["z2"][0].astype(np.float64)
    wb = inp["w_b"].astype(np.float64)
    for h in range(H):
        s_h = math.sqrt(float(inp["gamma"][h]) * wC / 2.0)   # s_h^2 = gamma w_C / 2
        qa = [inp["q"][0, :, h].astype(np.float64) / math.sqrt(C)]
        ka = [inp["k"][0, :, h].astype(np.float64)]
        for p in range(Pqk):
            qa.append(-_meet_phi(Qg[:, h, p], s_h))
            ka.append(_meet_psi(Kg[:, h, p], s_h))
        for r in range(R):
            qa.append(wb[:, h][None, :] * z1[:, r, :])
            ka.append(z2[:, r, :])
        Q = np.concatenate(qa, axis=1)[None]
        K = np.concatenate(ka, axis=1)[None]
        V = np.concatenate([inp["v"][0, :, h].astype(np.float64), Vg[:, h].reshape(L, -1)]
                           + [z2[:, r, :] for r in range(R)], axis=1)[None]
        o = _sdpa(Q, K, V, scale=wL)[0]                      # rho_h = w_L
        np.testing.assert_allclose(out["s"][0, :, h], o[:, :C], rtol=0, atol=1e-11)
        og = o[:, C:C + 3 * Pv].reshape(L, Pv, 3)
        loc = np.einsum("iyx,ipy->ipx", rot, og - trans[:, None, :])
        np.testing.assert_allclose(out["pts"][0, :, h], loc, rtol=0, atol=1e-10)
        np.testing.assert_allclose(out["pts_norm"][0, :, h], np.linalg.norm(loc, axis=-1),
                                   rtol=0, atol=1e-10)
        zo = o[:, C + 3 * Pv:].reshape(L, R, Cz)
        np.testing.assert_allclose(out["pair"][0, :, h], (z1 * zo).sum(1), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# invariances
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 7])
def test_se3_invariance(seed):
    inp = _inp(seed=seed)
    base = ipa_forward(inp)
    rng = np.random.default_rng(100 + seed)
    Rg = _rand_rot(rng)
    tg = rng.normal(0.0, 100.0, size=3)
    moved = dict(inp)
    moved["rot"] = np.einsum("xy,blyz->blxz", Rg, inp["rot"].astype(np.float64))
    moved["trans"] = np.einsum("xy,bly->blx", Rg, inp["trans"].astype(np.float64)) + tg
    out = ipa_forward(moved)
    for key in base:
        np.testing.assert_allclose(out[key], base[key], rtol=0, atol=1e-10, err_msg=key)


def test_permutation_equivariance():
    inp = _inp(seed=5)
    base = ipa_forward(inp)
    perm = np.random.default_rng(9).permutation(inp["dims"]["L"])
    moved = dict(inp)
    for key in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "mask"):
        moved[key] = inp[key][:, perm]
    out = ipa_forward(moved)
    for key in base:
        np.testing.assert_allclose(out[key], base[key][:, perm], rtol=0, atol=1e-12, err_msg=key)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_single_residue_closed_form():
    """L = 1: attention is 1 on the residue itself, so every value comes back
    unchanged in its own frame."""
    w = TINY.with_(L=1)
    inp = _inp(w, seed=2)
    out = ipa_forward(inp)
    np.testing.assert_allclose(out["s"], inp["v"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["pts"], inp["v_pts"], rtol=0, atol=1e-5)  # frames are fp32
    np.testing.assert_allclose(out["pts_norm"], np.linalg.norm(inp["v_pts"].astype(np.float64), axis=-1),
                               rtol=0, atol=1e-5)
    z = (inp["z1"].astype(np.float64) * inp["z2"].astype(np.float64)).sum(axis=2)  # [B,1,Cz]
    np.testing.assert_allclose(out["pair"], np.broadcast_to(z[:, :, None, :], out["pair"].shape),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [0.5, 1.5, 3.0])
def test_two_residue_distance_closed_form(D):
    """Two residues with identity frames D apart, zero local points, q = k = 0,
    W_b = 0: the only logit difference is the point term
    -w_L gamma w_C / 2 * Pqk * D^2, so a_12 = sigmoid(of it)."""
    w = TINY.with_(L=2, H=2)
    inp = _inp(w, seed=4)
    H, Pqk = w.H, w.Pqk
    inp["rot"] = np.broadcast_to(np.eye(3, dtype=np.float32), (1, 2, 3, 3)).copy()
    inp["trans"] = np.array([[[0.0, 0.0, 0.0], [D, 0.0, 0.0]]], np.float32)
    for key in ("q", "k", "q_pts", "k_pts"):
        inp[key] = np.zeros_like(inp[key])
    inp["w_b"] = np.zeros_like(inp["w_b"])
    out = ipa_forward(inp)
    for h in range(H):
        x = -inp["w_L"] * float(inp["gamma"][h]) * inp["w_C"] / 2.0 * Pqk * D * D
        a12 = 1.0 / (1.0 + math.exp(-x))
        v = inp["v"][0, :, h].astype(np.float64)
        expect = (1 - a12) * v[0] + a12 * v[1]
        np.testing.assert_allclose(out["s"][0, 0, h], expect, rtol=0, atol=1e-12)
        # points: sum_j a (R_j v + t_j) - t_0 with identity frames
        g = (1 - a12) * inp["v_pts"][0, 0, h].astype(np.float64) + a12 * (
            inp["v_pts"][0, 1, h].astype(np.float64) + np.array([D, 0.0, 0.0]))
        np.testing.assert_allclose(out["pts"][0, 0, h], g, rtol=0, atol=1e-6)


def test_uniform_attention_pair_closed_form():
    """q = k = 0, gamma = 0, W_b = 0 give uniform attention 1/n; then
    o_pair_i = sum_r z1_ir * mean_j z2_jr and o_pts = R_i^T(mean_j Vg_j - t_i)."""
    inp = _inp(seed=6)
    H = inp["dims"]["H"]
    for key in ("q", "k"):
        inp[key] = np.zeros_like(inp[key])
    inp["gamma"] = np.zeros(H, np.float32)
    inp["w_b"] = np.zeros_like(inp["w_b"])
    out = ipa_forward(inp)
    z1 = inp["z1"][0].astype(np.float64)
    z2m = inp["z2"][0].astype(np.float64).mean(axis=0)          # [R,Cz]
    expect = (z1 * z2m[None]).sum(axis=1)                        # [L,Cz]
    np.testing.assert_allclose(out["pair"][0], np.broadcast_to(expect[:, None], out["pair"][0].shape),
                               rtol=0, atol=1e-12)
    rot, trans = inp["rot"][0].astype(np.float64), inp["trans"][0].astype(np.float64)
    vg = to_global(rot, trans, inp["v_pts"][0].astype(np.float64)).mean(axis=0)   # [H,P,3]
    loc = np.einsum("iyx,ihpy->ihpx", rot, vg[None] - trans[:, None, None, :])
    np.testing.assert_allclose(out["pts"][0], loc, rtol=0, atol=1e-10)


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------

def test_masked_rows_exact_positive_zero_and_padding_ignored():
    w = WORKLOADS["ragged_batch"].with_(B=4, L=40, H=2, Cz=16, ragged=(5, 40), dtype="fp32")
    inp = make_inputs(w, seed=11)
    out = ipa_forward(inp)
    mask = inp["mask"].astype(bool)
    for key, o in out.items():
        m = ~mask
        sel = o[m]
        assert np.all(sel == 0.0) and not np.any(np.signbit(sel)), key
    # padded == unpadded: each sample alone on its valid prefix
    for b in range(w.B):
        n = int(inp["lengths"][b])
        sub = {k: (v[b:b + 1, :n] if isinstance(v, np.ndarray) and v.ndim >= 2 and v.shape[:2] == (w.B, w.L) else v)
               for k, v in inp.items()}
        sub["dims"] = dict(inp["dims"], B=1, L=n)
        sub["mask"] = np.ones((1, n), np.uint8)
        ref = ipa_forward(sub)
        for key in out:
            np.testing.assert_allclose(out[key][b, :n], ref[key][0], rtol=0, atol=1e-12, err_msg=key)


def test_scattered_mask_equals_valid_residues_alone():
    """A non-prefix mask (fully masked interior blocks, lone valid residues,
    masked first and last residues, an all-masked and a one-residue batch
    element): every valid row equals the oracle run on that batch element's
    valid residues alone, in order; masked rows are +0.0."""
    w = WORKLOADS["tiny_fp32"].with_(B=5, L=200, H=2, C=4, Pqk=2, Pv=3, R=1, Cz=8, mask="scatter")
    inp = make_inputs(w, seed=13)
    out = ipa_forward(inp)
    mask = inp["mask"].astype(bool)
    assert not mask[2].any() and mask[3].sum() == 1 and not mask[0, 0] and not mask[0, -1]
    for key, o in out.items():
        sel = o[~mask]
        assert np.all(sel == 0.0) and not np.any(np.signbit(sel)), key
    for b in range(w.B):
        idx = np.flatnonzero(mask[b])
        if idx.size == 0:
            continue
        sub = {k: (v[b:b + 1][:, idx] if isinstance(v, np.ndarray) and v.ndim >= 2 and v.shape[:2] == (w.B, w.L) else v)
               for k, v in inp.items()}
        sub["dims"] = dict(inp["dims"], B=1, L=int(idx.size))
        sub["mask"] = np.ones((1, idx.size), np.uint8)
        ref = ipa_forward(sub)
        for key in out:
            np.testing.assert_allclose(out[key][b, idx], ref[key][0], rtol=0, atol=1e-12, err_msg=key)


def test_to_global_closed_form():
    """A quarter turn about z maps local (x, y, z) to (-y, x, z); the frame
    origin is added after the turn."""
    rot = np.array([[[0.0, -1.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 1.0]]])
    trans = np.array([[10.0, -2.0, 0.5]])
    pts = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 1, 3)
    g = to_global(rot, trans, pts)
    np.testing.assert_allclose(g.reshape(3), [10.0 - 2.0, -2.0 + 1.0, 0.5 + 3.0], rtol=0, atol=1e-15)


def test_garbage_in_padding_does_not_change_valid_rows():
    w = WORKLOADS["ragged_batch"].with_(B=2, L=32, H=2, Cz=16, ragged=(10, 30), dtype="fp32")
    inp = make_inputs(w, seed=12)
    base = ipa_forward(inp)
    rng = np.random.default_rng(5)
    pad = inp["mask"] == 0
    moved = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    for key in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2", "rot", "trans"):
        a = moved[key]
        a[pad] = rng.normal(0, 1e3, size=a[pad].shape).astype(a.dtype)
    out = ipa_forward(moved)
    for key in base:
        np.testing.assert_array_equal(out[key][~pad], base[key][~pad])


# ----------------------------------------------------------------------------
# agreement of the three fp64 forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_agrees(seed):
    w = TINY.with_(L=6, H=2, C=4, Pqk=2, Pv=3, Cz=8)
    inp = make_inputs(w, seed=seed)
    a, b = ipa_forward(inp), ipa_bruteforce(inp)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=0, atol=1e-12, err_msg=key)


@pytest.mark.parametrize("G", [4, 16, 64])
def test_lifted_form_agrees(G):
    w = WORKLOADS["ragged_batch"].with_(B=3, L=100, H=2, Cz=16, ragged=(20, 100), step=3.8)
    inp = make_inputs(w, seed=3)
    a, c = ipa_forward(inp), ipa_lifted(inp, G=G)
    for key in a:
        scale = max(1.0, float(np.abs(a[key]).max()))
        np.testing.assert_allclose(c[key], a[key], rtol=0, atol=1e-12 * scale * 10, err_msg=key)


def test_lifted_form_any_centres():
    """Block centres only move the expansion point: arbitrary centres give the
    same result (the offsets are exact algebra)."""
    w = TINY.with_(L=40)
    inp = make_inputs(w, seed=8)
    a = ipa_forward(inp)
    cen = np.random.default_rng(0).normal(0, 50.0, size=(1, 5, 3))
    c = ipa_lifted(inp, G=8, centres=cen)
    for key in a:
        np.testing.assert_allclose(c[key], a[key], rtol=0, atol=1e-10, err_msg=key)


# ----------------------------------------------------------------------------
# generator sanity (shared seeded inputs, no method arithmetic)
# ----------------------------------------------------------------------------

def test_generators():
    inp = make_inputs(WORKLOADS["single_chain"])
    R = inp["rot"][0].astype(np.float64)
    np.testing.assert_allclose(np.einsum("lxy,lzy->lxz", R, R), np.broadcast_to(np.eye(3), R.shape), atol=1e-6)
    np.testing.assert_allclose(np.linalg.det(R), 1.0, atol=1e-5)
    t = inp["trans"][0].astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(np.diff(t, axis=0), axis=1), 3.8, atol=1e-4)
    np.testing.assert_allclose(t.mean(axis=0), 0.0, atol=1e-4)
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32) * 37.0
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(x), ref)
    assert np.array_equal(round_to_bf16(inp["q"]), inp["q"])


# ----------------------------------------------------------------------------
# planted mistakes: each one must be caught by a pin above
# ----------------------------------------------------------------------------

def _run_pins(monkeypatch_target):
    failures = 0
    for fn in (test_single_residue_closed_form,
               lambda: test_two_residue_distance_closed_form(1.5),
               lambda: test_meet_lifting_identity_through_library_attention(0),
               test_uniform_attention_pair_closed_form,
               lambda: test_se3_invariance(0)):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def test_planted_transposed_rotation_is_caught(monkeypatch):
    def bad(rot_b, trans_b, pts_b):
        return np.einsum("lyx,lhpy->lhpx", rot_b, pts_b) + trans_b[:, None, None, :]
    monkeypatch.setattr(oracle_mod, "to_global", bad)
    assert _run_pins(oracle_mod) > 0


def test_planted_distance_sign_is_caught(monkeypatch):
    orig = oracle_mod.ipa_forward

    def bad(inp, rows=None, row_block=None):
        flipped = dict(inp)
        flipped["gamma"] = -np.asarray(inp["gamma"])
        return orig(flipped, rows=rows, row_block=row_block)
    monkeypatch.setattr(oracle_mod, "ipa_forward", bad)
    monkeypatch.setitem(globals(), "ipa_forward", bad)
    assert _run_pins(oracle_mod) > 0


def test_planted_dropped_pair_bias_is_caught(monkeypatch):
    orig = oracle_mod.ipa_forward

    def bad(inp, rows=None, row_block=None):
        dropped = dict(inp)
        dropped["w_b"] = np.zeros_like(inp["w_b"])
        return orig(dropped, rows=rows, row_block=row_block)
    monkeypatch.setitem(globals(), "ipa_forward", bad)
    assert _run_pins(oracle_mod) > 0
