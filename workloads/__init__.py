"""Seeded synthetic inputs for invariant point attention (IPA) workloads.

This module only draws and shapes random inputs. It holds none of the
attention arithmetic, so both the fp64 oracle and the GPU path can take
their inputs from it without sharing any of the method.

Input recipe (one ``numpy.random.default_rng(seed)`` per call, draws in a
fixed order: quaternions, chain steps, q, k, v, q_pts, k_pts, v_pts, z1, z2,
gamma logits, pair-bias weights, lengths, padding garbage):

* rotations: a Gaussian quaternion normalised to unit length, turned into a
  rotation matrix that maps local column vectors to the global frame
  (Haar-uniform on SO(3));
* translations: a chain that starts at the origin and takes steps of fixed
  length (3.8 A for protein-like chains, 5.9 A for RNA-like ones) in
  uniformly random directions, then is centred on its mean;
* per-head scalars and local points ~ N(0, 1);
* pair factors z1, z2 ~ N(0, 1) / sqrt(c_z) (standard deviation 1/sqrt(c_z));
* gamma = softplus(N(0, 1)) per head, pair-bias weights W_b ~ N(0, 1);
* ragged batches: true lengths uniform in [lo, hi], a prefix validity mask,
  and padded rows filled with finite garbage (N(0, 10^2) features,
  non-orthogonal N(0, 1) "rotations", translations uniform in +-1e3);
* scattered masks (``mask="scatter"``): a non-prefix validity mask drawn
  after everything above from a generator of its own (``scatter_mask``),
  with the same finite garbage in every masked row; the chain runs through
  all L residues and is centred on its valid ones.

For the bf16-storage workloads every per-residue feature tensor (q, k, v,
points, z1, z2) is rounded to bfloat16 (round to nearest even) here, before
either side sees it; frames, W_b and gamma stay float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import numpy as np


@dataclass(frozen=True)
class IPAWorkload:
    name: str
    B: int
    L: int
    H: int
    C: int = 16
    Pqk: int = 4
    Pv: int = 8
    R: int = 2
    Cz: int = 128
    dtype: str = "bf16"          # storage of q, k, v, points, z1, z2
    step: float = 3.8            # chain step length in Angstrom
    ragged: tuple | None = None  # (lo, hi) true lengths, prefix mask
    seed: int = 0
    mask: str | None = None      # "scatter": non-prefix mask (scatter_mask)

    def dims(self) -> dict:
        return dict(B=self.B, L=self.L, H=self.H, C=self.C, Pqk=self.Pqk,
                    Pv=self.Pv, R=self.R, Cz=self.Cz)

    def with_(self, **kw) -> "IPAWorkload":
        d = asdict(self)
        d.update(kw)
        return IPAWorkload(**d)


# The five workload families the method is measured on.
WORKLOADS = {
    "tiny_fp32": IPAWorkload("tiny_fp32", B=1, L=64, H=12, Cz=16, dtype="fp32"),
    "single_chain": IPAWorkload("single_chain", B=1, L=512, H=12, Cz=128),
    "long_chain_2048": IPAWorkload("long_chain_2048", B=1, L=2048, H=12, Cz=128),
    "long_chain_4096": IPAWorkload("long_chain_4096", B=1, L=4096, H=12, Cz=128),
    "ragged_batch": IPAWorkload("ragged_batch", B=32, L=128, H=8, Cz=64,
                                step=5.9, ragged=(40, 128)),
    "very_long_8192": IPAWorkload("very_long_8192", B=1, L=8192, H=8, Cz=128),
    "very_long_16384": IPAWorkload("very_long_16384", B=1, L=16384, H=8, Cz=128),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(a.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _quat_to_rot(u: np.ndarray) -> np.ndarray:
    u = u / np.linalg.norm(u, axis=-1, keepdims=True)
    w, x, y, z = u[..., 0], u[..., 1], u[..., 2], u[..., 3]
    R = np.empty(u.shape[:-1] + (3, 3), dtype=np.float64)
    R[..., 0, 0] = 1 - 2 * (y * y + z * z)
    R[..., 0, 1] = 2 * (x * y - w * z)
    R[..., 0, 2] = 2 * (x * z + w * y)
    R[..., 1, 0] = 2 * (x * y + w * z)
    R[..., 1, 1] = 1 - 2 * (x * x + z * z)
    R[..., 1, 2] = 2 * (y * z - w * x)
    R[..., 2, 0] = 2 * (x * z - w * y)
    R[..., 2, 1] = 2 * (y * z + w * x)
    R[..., 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def default_weights(Pqk: int) -> tuple[float, float]:
    """Default logit weights w_L = sqrt(1/3), w_C = sqrt(2 / (9 Pqk))."""
    return math.sqrt(1.0 / 3.0), math.sqrt(2.0 / (9.0 * Pqk))


def scatter_mask(B: int, L: int, rng: np.random.Generator) -> np.ndarray:
    """A non-prefix validity mask [B, L] (uint8) with the structures a mask
    can take: batch element 0 has its first and last residues masked, whole
    interior 64-residue blocks masked (one of them holding a single valid
    residue) and the rest kept with probability ~0.75; element 1 has only
    its last residue masked and sparse partial blocks (keep ~0.35);
    element 2 is masked entirely; element 3 has exactly one valid residue;
    further elements draw a keep rate in [0.2, 0.95] and mask their first
    or last residue at random."""
    m = np.zeros((B, L), dtype=np.uint8)
    nblk = (L + 63) // 64
    for b in range(B):
        if b == 2:
            continue
        if b == 3:
            m[b, rng.integers(L)] = 1
            continue
        keep = 0.75 if b == 0 else 0.35 if b == 1 else rng.uniform(0.2, 0.95)
        row = rng.random(L) < keep
        if nblk >= 3 and b != 1:
            inner = np.arange(1, nblk - 1)
            full = rng.choice(inner, size=max(1, len(inner) // 3), replace=False)
            for J in full:
                row[64 * J:min(L, 64 * J + 64)] = False
            if len(full) >= 2:
                J = int(full[0])
                row[64 * J + rng.integers(min(64, L - 64 * J))] = True
        if b == 0:
            row[0] = row[-1] = False
        elif b == 1:
            row[0], row[-1] = True, False
        else:
            if rng.random() < 0.5:
                row[0] = False
            if rng.random() < 0.5:
                row[-1] = False
        if not row.any():
            row[rng.integers(L)] = True
        m[b] = row
    return m


def make_inputs(w: IPAWorkload, seed: int | None = None) -> dict:
    """Draw one seeded input set for workload ``w``.

    Returns a dict of numpy arrays: float32 features (bf16-representable for
    bf16 workloads), float32 frames, uint8 mask, plus scalars and metadata.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, L, H, C, Pqk, Pv, R, Cz = w.B, w.L, w.H, w.C, w.Pqk, w.Pv, w.R, w.Cz

    quat = rng.standard_normal((B, L, 4))
    steps = rng.standard_normal((B, L, 3))
    q = rng.standard_normal((B, L, H, C))
    k = rng.standard_normal((B, L, H, C))
    v = rng.standard_normal((B, L, H, C))
    q_pts = rng.standard_normal((B, L, H, Pqk, 3))
    k_pts = rng.standard_normal((B, L, H, Pqk, 3))
    v_pts = rng.standard_normal((B, L, H, Pv, 3))
    z1 = rng.standard_normal((B, L, R, Cz)) / math.sqrt(Cz)
    z2 = rng.standard_normal((B, L, R, Cz)) / math.sqrt(Cz)
    gamma = _softplus(rng.standard_normal(H))
    w_b = rng.standard_normal((Cz, H))

    if w.ragged is not None:
        lo, hi = w.ragged
        lengths = rng.integers(lo, hi + 1, size=B)
    else:
        lengths = np.full(B, L, dtype=np.int64)

    rot = _quat_to_rot(quat)
    trans = np.zeros((B, L, 3))
    mask = np.zeros((B, L), dtype=np.uint8)
    for b in range(B):
        n = int(lengths[b])
        mask[b, :n] = 1
        g = steps[b, :n]
        g = g / np.linalg.norm(g, axis=-1, keepdims=True)
        x = np.zeros((n, 3))
        if n > 1:
            x[1:] = np.cumsum(w.step * g[1:], axis=0)
        trans[b, :n] = x - x.mean(axis=0)

    if w.mask == "scatter":
        if w.ragged is not None:
            raise ValueError("a workload takes either ragged lengths or a scattered mask")
        # the mask and its garbage come from a generator of their own, so the
        # draws above are those of the unmasked workload
        rng = np.random.default_rng([w.seed if seed is None else seed, 0x5CA7])
        mask = scatter_mask(B, L, rng)
        lengths = mask.sum(axis=1).astype(np.int64)
        for b in range(B):
            vb = mask[b] != 0
            if vb.any():
                trans[b] -= trans[b][vb].mean(axis=0)
    if w.ragged is not None or w.mask == "scatter":
        # finite garbage in every padded row
        pad = mask == 0
        npad = int(pad.sum())
        if npad:
            def garb(shape):
                return 10.0 * rng.standard_normal((npad,) + shape)
            q[pad] = garb((H, C)); k[pad] = garb((H, C)); v[pad] = garb((H, C))
            q_pts[pad] = garb((H, Pqk, 3)); k_pts[pad] = garb((H, Pqk, 3))
            v_pts[pad] = garb((H, Pv, 3))
            z1[pad] = garb((R, Cz)); z2[pad] = garb((R, Cz))
            rot[pad] = rng.standard_normal((npad, 3, 3))
            trans[pad] = rng.uniform(-1e3, 1e3, size=(npad, 3))

    feats = dict(q=q, k=k, v=v, q_pts=q_pts, k_pts=k_pts, v_pts=v_pts, z1=z1, z2=z2)
    for name, a in feats.items():
        a32 = a.astype(np.float32)
        feats[name] = round_to_bf16(a32) if w.dtype == "bf16" else a32

    w_L, w_C = default_weights(Pqk)
    out = dict(feats)
    out.update(
        rot=rot.astype(np.float32), trans=trans.astype(np.float32),
        gamma=gamma.astype(np.float32), w_b=w_b.astype(np.float32),
        mask=mask, lengths=lengths.astype(np.int64),
        w_L=w_L, w_C=w_C, dtype=w.dtype, dims=w.dims(), workload=w.name,
        has_mask=w.ragged is not None or w.mask == "scatter",
    )
    return out


def stress_pair(inp: dict) -> dict:
    """Pair-stress variant: z1, z2 rescaled to unit variance so that the pair
    bias and pair output are O(1) and a pair-path error is visible."""
    out = dict(inp)
    Cz = inp["dims"]["Cz"]
    for name in ("z1", "z2"):
        a = inp[name].astype(np.float32) * np.float32(math.sqrt(Cz))
        out[name] = round_to_bf16(a) if inp["dtype"] == "bf16" else a
    return out


# ----------------------------------------------------------------------------
# backbone atoms (input of the frame construction)
# ----------------------------------------------------------------------------

def make_backbone(B: int, L: int, seed: int = 0, step: float = 3.8) -> dict:
    """Seeded backbone atoms N, C-alpha, C as float32 [B, L, 3] arrays.

    C-alpha atoms follow the same centred chain as the frame translations
    (fixed steps of ``step`` A in uniformly random directions). Around each
    C-alpha, C sits 1.52 A away in a uniformly random direction and N 1.46 A
    away at an angle of 111 degrees to it, turned by a uniformly random
    angle about the C-alpha -> C axis (protein-like bond lengths and angle;
    never collinear). Draw order: chain steps, C directions, N turn angles.
    """
    rng = np.random.default_rng(seed)
    steps = rng.standard_normal((B, L, 3))
    cdir = rng.standard_normal((B, L, 3))
    turn = rng.uniform(0.0, 2.0 * math.pi, size=(B, L))
    g = steps / np.linalg.norm(steps, axis=-1, keepdims=True)
    ca = np.zeros((B, L, 3))
    ca[:, 1:] = np.cumsum(step * g[:, 1:], axis=1)
    ca -= ca.mean(axis=1, keepdims=True)
    u = cdir / np.linalg.norm(cdir, axis=-1, keepdims=True)
    # two unit vectors orthogonal to u
    a = np.where(np.abs(u[..., :1]) < 0.9, np.array([1.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0]))
    p = np.cross(u, a)
    p /= np.linalg.norm(p, axis=-1, keepdims=True)
    r = np.cross(u, p)
    ang = math.radians(111.0)
    ndir = math.cos(ang) * u + math.sin(ang) * (np.cos(turn)[..., None] * p + np.sin(turn)[..., None] * r)
    c = ca + 1.52 * u
    n = ca + 1.46 * ndir
    return dict(n=n.astype(np.float32), ca=ca.astype(np.float32), c=c.astype(np.float32))


# ----------------------------------------------------------------------------
# distance-penalised attention over one point per residue
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class MeetWorkload:
    name: str
    B: int
    L: int
    H: int
    C: int = 16
    dtype: str = "bf16"          # storage of q, k, v
    step: float = 3.8
    ragged: tuple | None = None
    seed: int = 0
    mask: str | None = None      # "scatter": non-prefix mask (scatter_mask)

    def dims(self) -> dict:
        return dict(B=self.B, L=self.L, H=self.H, C=self.C)

    def with_(self, **kw) -> "MeetWorkload":
        d = asdict(self)
        d.update(kw)
        return MeetWorkload(**d)


MEET_WORKLOADS = {
    "meet_tiny_fp32": MeetWorkload("meet_tiny_fp32", B=1, L=64, H=4, dtype="fp32"),
    "meet_chain_512": MeetWorkload("meet_chain_512", B=1, L=512, H=12),
    "meet_chain_2048": MeetWorkload("meet_chain_2048", B=1, L=2048, H=12),
    "meet_ragged": MeetWorkload("meet_ragged", B=8, L=128, H=8, ragged=(40, 128)),
}


def make_meet_inputs(w: MeetWorkload, seed: int | None = None) -> dict:
    """Draw one seeded input set for a distance-attention workload.

    Draw order: chain steps, q, k, v, rho logits, s logits, lengths, padding
    garbage. x is the centred chain of the IPA recipe; q, k, v ~ N(0, 1);
    rho_h = softplus(N(0, 1)) / sqrt(C); s_h = 0.2 softplus(N(0, 1)) (per
    A). Ragged batches get a prefix mask and finite garbage in padded rows;
    ``mask="scatter"`` draws a non-prefix mask (``scatter_mask``) and its
    garbage from a generator of their own after everything else.
    bf16 workloads round q, k, v to bfloat16 here; x, rho, s stay float32.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, L, H, C = w.B, w.L, w.H, w.C
    steps = rng.standard_normal((B, L, 3))
    q = rng.standard_normal((B, L, H, C))
    k = rng.standard_normal((B, L, H, C))
    v = rng.standard_normal((B, L, H, C))
    rho = _softplus(rng.standard_normal(H)) / math.sqrt(C)
    s = 0.2 * _softplus(rng.standard_normal(H))
    if w.ragged is not None:
        lo, hi = w.ragged
        lengths = rng.integers(lo, hi + 1, size=B)
    else:
        lengths = np.full(B, L, dtype=np.int64)
    x = np.zeros((B, L, 3))
    mask = np.zeros((B, L), dtype=np.uint8)
    for b in range(B):
        n = int(lengths[b])
        mask[b, :n] = 1
        g = steps[b, :n] / np.linalg.norm(steps[b, :n], axis=-1, keepdims=True)
        xb = np.zeros((n, 3))
        if n > 1:
            xb[1:] = np.cumsum(w.step * g[1:], axis=0)
        x[b, :n] = xb - xb.mean(axis=0)
    if w.mask == "scatter":
        if w.ragged is not None:
            raise ValueError("a workload takes either ragged lengths or a scattered mask")
        rng = np.random.default_rng([w.seed if seed is None else seed, 0x5CA7])
        mask = scatter_mask(B, L, rng)
        lengths = mask.sum(axis=1).astype(np.int64)
        for b in range(B):
            vb = mask[b] != 0
            if vb.any():
                x[b] -= x[b][vb].mean(axis=0)
    if w.ragged is not None or w.mask == "scatter":
        pad = mask == 0
        npad = int(pad.sum())
        if npad:
            q[pad] = 10.0 * rng.standard_normal((npad, H, C))
            k[pad] = 10.0 * rng.standard_normal((npad, H, C))
            v[pad] = 10.0 * rng.standard_normal((npad, H, C))
            x[pad] = rng.uniform(-1e3, 1e3, size=(npad, 3))
    feats = {}
    for name, a in (("q", q), ("k", k), ("v", v)):
        a32 = a.astype(np.float32)
        feats[name] = round_to_bf16(a32) if w.dtype == "bf16" else a32
    out = dict(feats)
    out.update(x=x.astype(np.float32), rho=rho.astype(np.float32), s=s.astype(np.float32),
               mask=mask, lengths=lengths.astype(np.int64), dtype=w.dtype, dims=w.dims(),
               workload=w.name, has_mask=w.ragged is not None or w.mask == "scatter")
    return out


# ----------------------------------------------------------------------------
# direction-and-distance attention
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class DirDistWorkload:
    name: str
    B: int
    N: int
    H: int
    M: int = 8                   # value vectors per head
    Cout: int = 384
    step: float = 3.8
    ragged: tuple | None = None
    pair_mask: str | None = None  # None, "full" [B,H,N,N], "per_head" [1,H,N,N], "shared" [N,N]
    bias: bool = True
    seed: int = 0

    def dims(self) -> dict:
        return dict(B=self.B, N=self.N, H=self.H, M=self.M, Cout=self.Cout)

    def with_(self, **kw) -> "DirDistWorkload":
        d = asdict(self)
        d.update(kw)
        return DirDistWorkload(**d)


DIRDIST_WORKLOADS = {
    "dd_tiny_fp32": DirDistWorkload("dd_tiny_fp32", B=2, N=37, H=3, M=2, Cout=5,
                                    ragged=(20, 37), pair_mask="full"),
    "dd_chain_512": DirDistWorkload("dd_chain_512", B=1, N=512, H=12),
    "dd_chain_2048": DirDistWorkload("dd_chain_2048", B=1, N=2048, H=12),
    "dd_ragged": DirDistWorkload("dd_ragged", B=8, N=128, H=8, M=4, Cout=64,
                                 ragged=(40, 128), pair_mask="per_head"),
}


def make_dirdist_inputs(w: DirDistWorkload, seed: int | None = None) -> dict:
    """Draw one seeded input set for a direction-and-distance workload.

    Draw order: quaternions, chain steps, q_direction, k_direction, q_point,
    k_point, values, direction_scale, distance_scale, output_weight,
    output_bias, lengths, pair mask, padding garbage. Frames follow the IPA
    recipe (Haar rotations, centred chain of fixed step); local directions,
    points and values ~ N(0, 1); the two per-head scales are raw N(0, 1)
    logits (softplus is part of the method); output_weight ~
    N(0, 1) / sqrt(3 H M), output_bias ~ N(0, 1); a pair mask keeps each edge
    with probability 0.9. All arrays float32; masks uint8.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, N, H, M, Cout = w.B, w.N, w.H, w.M, w.Cout
    quat = rng.standard_normal((B, N, 4))
    steps = rng.standard_normal((B, N, 3))
    qdir = rng.standard_normal((B, N, H, 3))
    kdir = rng.standard_normal((B, N, H, 3))
    qpt = rng.standard_normal((B, N, H, 3))
    kpt = rng.standard_normal((B, N, H, 3))
    val = rng.standard_normal((B, N, H, M, 3))
    dsc = rng.standard_normal(H)
    ssc = rng.standard_normal(H)
    W = rng.standard_normal((H * M * 3, Cout)) / math.sqrt(3 * H * M)
    bias = rng.standard_normal(Cout)
    if w.ragged is not None:
        lo, hi = w.ragged
        if not 1 <= lo <= hi <= N:
            raise ValueError(f"ragged lengths {w.ragged} must lie in [1, N={N}]")
        lengths = rng.integers(lo, hi + 1, size=B)
    else:
        lengths = np.full(B, N, dtype=np.int64)
    pm = None
    if w.pair_mask == "full":
        pm = (rng.random((B, H, N, N)) < 0.9).astype(np.uint8)
    elif w.pair_mask == "per_head":
        pm = (rng.random((1, H, N, N)) < 0.9).astype(np.uint8)
    elif w.pair_mask == "shared":
        pm = (rng.random((N, N)) < 0.9).astype(np.uint8)
    rot = _quat_to_rot(quat)
    trans = np.zeros((B, N, 3))
    fmask = np.zeros((B, N), dtype=np.uint8)
    for b in range(B):
        n = int(lengths[b])
        fmask[b, :n] = 1
        g = steps[b, :n] / np.linalg.norm(steps[b, :n], axis=-1, keepdims=True)
        x = np.zeros((n, 3))
        if n > 1:
            x[1:] = np.cumsum(w.step * g[1:], axis=0)
        trans[b, :n] = x - x.mean(axis=0)
    if w.ragged is not None:
        pad = fmask == 0
        npad = int(pad.sum())
        if npad:
            qdir[pad] = 10.0 * rng.standard_normal((npad, H, 3))
            kdir[pad] = 10.0 * rng.standard_normal((npad, H, 3))
            qpt[pad] = 10.0 * rng.standard_normal((npad, H, 3))
            kpt[pad] = 10.0 * rng.standard_normal((npad, H, 3))
            val[pad] = 10.0 * rng.standard_normal((npad, H, M, 3))
            rot[pad] = rng.standard_normal((npad, 3, 3))
            trans[pad] = rng.uniform(-1e3, 1e3, size=(npad, 3))
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return dict(
        rot=f32(rot), trans=f32(trans), q_direction=f32(qdir), k_direction=f32(kdir),
        q_point=f32(qpt), k_point=f32(kpt), values=f32(val),
        direction_scale=f32(dsc), distance_scale=f32(ssc),
        output_weight=f32(W), output_bias=f32(bias) if w.bias else None,
        frame_mask=fmask, pair_mask=pm, lengths=lengths.astype(np.int64),
        dims=w.dims(), workload=w.name,
    )


# ----------------------------------------------------------------------------
# the full layer around the attention
# ----------------------------------------------------------------------------
def make_layer_inputs(w: IPAWorkload, c_s: int = 384, seed: int | None = None) -> dict:
    """Draw one seeded input set for the IPA layer with single-representation
    width c_s: frames, mask, W_b and gamma as ``make_inputs(w)``; then
    s ~ N(0, 1) [B,L,c_s]; the input map W_in [c_s, Nin] with columns
    ~ N(0, 1/c_s) (projected features of unit variance; the pair-factor
    columns scaled by 1/sqrt(c_z), as in the IPA recipe), b_in ~ N(0, 0.1^2);
    the readout W_out [Nout, c_s] ~ N(0, 1/Nout), b_out ~ N(0, 1). Column
    blocks of W_in: q, k, v [H C each], q_pts, k_pts [H Pqk 3], v_pts
    [H Pv 3], z1, z2 [R c_z]; rows of W_out: o_s [H C], o_pts [H Pv 3],
    o_norm [H Pv], o_pair [H c_z]. float32 throughout.
    """
    base = make_inputs(w, seed=seed)
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    B, L, H, C, Pqk, Pv, R, Cz = w.B, w.L, w.H, w.C, w.Pqk, w.Pv, w.R, w.Cz
    n_in = 3 * H * C + 3 * H * Pqk * 2 + 3 * H * Pv + 2 * R * Cz
    n_out = H * (C + 3 * Pv + Pv + Cz)
    s = rng.standard_normal((B, L, c_s))
    w_in = rng.standard_normal((c_s, n_in)) / math.sqrt(c_s)
    w_in[:, n_in - 2 * R * Cz:] /= math.sqrt(Cz)
    b_in = 0.1 * rng.standard_normal(n_in)
    w_out = rng.standard_normal((n_out, c_s)) / math.sqrt(n_out)
    b_out = rng.standard_normal(c_s)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return dict(s=f32(s), rot=base["rot"], trans=base["trans"], mask=base["mask"],
                has_mask=base["has_mask"], w_in=f32(w_in), b_in=f32(b_in), w_b=base["w_b"],
                gamma=base["gamma"], w_L=base["w_L"], w_C=base["w_C"], w_out=f32(w_out),
                b_out=f32(b_out), dims=w.dims(), c_s=c_s, dtype=w.dtype, workload=w.name)
