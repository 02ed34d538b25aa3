"""GPU parity of the full IPA layer (ipa_layer_forward) against the fp64
layer oracle, through the C ABI.

Tolerance on the output, relative to its scale (max(1, max |reference|)):
fp32 storage 1e-4 (fp32 projections and readout, sums of a few hundred
terms, around the fp32 attention); bf16 storage 3e-2 (the attention's own
bf16 bound; a projected feature that lands on a bf16 rounding boundary may
round the other way on the two sides, one bf16 ulp, well inside it).
Masked rows must be exact +0.0.
"""

import numpy as np
import pytest
import torch

from oracle import ipa_layer
from workloads import WORKLOADS, make_layer_inputs

pytestmark = pytest.mark.gpu


def _gpu(inp, device):
    from geometric_invariant_attention_amd import IPALayer
    d = inp["dims"]
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(inp[k]).to(device) for k in ("s", "rot", "trans", "w_in", "b_in", "w_b",
                                                          "gamma", "w_out", "b_out")}
    m = torch.from_numpy(inp["mask"]).to(device) if inp.get("has_mask") else None
    layer = IPALayer(**d, c_s=inp["c_s"], dtype=dt, device=device)
    y = layer(t["s"], t["rot"], t["trans"], t["w_in"], t["b_in"], t["w_b"], t["gamma"], t["w_out"],
              t["b_out"], mask=m, w_L=inp["w_L"], w_C=inp["w_C"])
    torch.cuda.synchronize()
    return y.cpu().numpy().copy()


def _check(w, device, c_s, tol, seed=0):
    print(f"[layer] {w.name} dims={w.dims()} c_s={c_s} dtype={w.dtype} seed={seed}", flush=True)
    inp = make_layer_inputs(w, c_s=c_s, seed=seed)
    got = _gpu(inp, device)
    ref = ipa_layer(inp)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max()) / max(1.0, float(np.abs(ref).max()))
    print(f"  rel error {err:.2e}", flush=True)
    assert err < tol, err
    return inp, got


@pytest.mark.parametrize("L,c_s", [(1, 8), (37, 24), (64, 96)])
def test_layer_fp32(device, L, c_s):
    _check(WORKLOADS["tiny_fp32"].with_(L=L, H=4), device, c_s, 1e-4, seed=L)


def test_layer_bf16_single_chain(device):
    _check(WORKLOADS["single_chain"].with_(L=200), device, 384, 3e-2)


@pytest.mark.parametrize("c_s", [24, 72])
def test_layer_bf16_narrow_readout(device, c_s):
    """bf16 storage with a narrow single representation: the split-path
    projection and readout on small output widths and a ragged row tail."""
    _check(WORKLOADS["single_chain"].with_(L=77, H=4), device, c_s, 3e-2, seed=c_s)


def test_layer_ragged_batch_masked_rows_zero(device):
    inp, got = _check(WORKLOADS["ragged_batch"].with_(B=4, L=70, ragged=(30, 70)), device, 128, 3e-2, seed=2)
    pad = inp["mask"] == 0
    assert np.all(got[pad] == 0) and not np.signbit(got[pad]).any()


def test_layer_no_biases(device):
    from geometric_invariant_attention_amd import IPALayer
    w = WORKLOADS["tiny_fp32"].with_(L=33, H=3)
    inp = make_layer_inputs(w, c_s=16, seed=5)
    d = inp["dims"]
    t = {k: torch.from_numpy(inp[k]).to(device) for k in ("s", "rot", "trans", "w_in", "w_b", "gamma", "w_out")}
    y = IPALayer(**d, c_s=16, dtype=torch.float32, device=device)(
        t["s"], t["rot"], t["trans"], t["w_in"], None, t["w_b"], t["gamma"], t["w_out"], None,
        w_L=inp["w_L"], w_C=inp["w_C"])
    torch.cuda.synchronize()
    inp["b_in"] = np.zeros_like(inp["b_in"])
    inp["b_out"] = np.zeros_like(inp["b_out"])
    ref = ipa_layer(inp)
    assert np.abs(y.cpu().numpy() - ref).max() / max(1.0, np.abs(ref).max()) < 1e-4


def test_layer_long_chain_2048_sampled_rows(device):
    """The layer at the benchmarked size (L = 2048, H = 12, c_z = 128,
    c_s = 384, bf16 attention), checked on sampled rows: tile edges and
    random rows; the oracle computes each output row from every residue's
    features and that row's attention alone."""
    w = WORKLOADS["long_chain_2048"]
    print(f"[layer] {w.name} dims={w.dims()} c_s=384 sampled rows", flush=True)
    inp = make_layer_inputs(w, c_s=384, seed=0)
    got = _gpu(inp, device)
    L = w.L
    edges = {i for t in range(0, L + 1, 64) for i in (t - 1, t) if 0 <= i < L}
    rng = np.random.default_rng(1)
    rows = np.array(sorted(edges | set(rng.choice(L, 16, replace=False).tolist()))[::2])
    ref = ipa_layer(inp, rows=rows)
    err = float(np.abs(got[:, rows] - ref).max()) / max(1.0, float(np.abs(ref).max()))
    print(f"  {len(rows)} rows, rel error {err:.2e}", flush=True)
    assert np.isfinite(got).all()
    assert err < 3e-2, err


def test_layer_unaligned_output_blocks(device):
    """H C = 15 and H Pv = 9 floats: the attention's output blocks would not
    start on 16-byte boundaries of the readout matrix, so the layer takes
    its packed-output-plus-gather path."""
    _check(WORKLOADS["tiny_fp32"].with_(L=45, H=3, C=5, Pv=3, Cz=8, R=1), device, 24, 1e-4, seed=6)


def test_layer_readout_split_along_rows(device):
    """A readout whose gathered operand spans 2^29 elements or more runs as
    several launches along its rows (the matrix kernels address an operand
    slice with 32-bit byte offsets). 500 copies of one fp32 chain of 512
    residues (H = 12, c_z = 128, R = 1) make 256000 rows x 2112 gathered
    columns, split into a launch
    of 254080 rows and one of 1920; the first and the last copy, which fall
    in different launches, are compared with the oracle on the one chain."""
    from geometric_invariant_attention_amd import IPALayer
    w1 = WORKLOADS["single_chain"].with_(dtype="fp32", R=1)   # fp32 storage: R c_z <= 128
    one = make_layer_inputs(w1, c_s=64, seed=13)
    copies = 500
    big = dict(one)
    for k in ("s", "rot", "trans", "mask"):
        big[k] = np.ascontiguousarray(np.repeat(one[k], copies, axis=0))
    d = dict(one["dims"], B=copies)
    assert d["B"] * d["L"] * d["H"] * (d["C"] + 4 * d["Pv"] + d["Cz"]) >= 2 ** 29
    print(f"[layer] {copies} copies of {w1.name} (fp32, c_s=64): readout split along rows", flush=True)
    t = {k: torch.from_numpy(big[k]).to(device) for k in ("s", "rot", "trans", "w_in", "b_in", "w_b",
                                                          "gamma", "w_out", "b_out")}
    m = torch.from_numpy(big["mask"]).to(device) if big.get("has_mask") else None
    layer = IPALayer(**d, c_s=64, dtype=torch.float32, device=device)
    y = layer(t["s"], t["rot"], t["trans"], t["w_in"], t["b_in"], t["w_b"], t["gamma"], t["w_out"],
              t["b_out"], mask=m, w_L=big["w_L"], w_C=big["w_C"])
    torch.cuda.synchronize()
    got = y[[0, copies - 1]].cpu().numpy()
    del y, layer, t
    ref = ipa_layer(one)[0]
    scale = max(1.0, float(np.abs(ref).max()))
    for c, g in zip((0, copies - 1), got):
        err = float(np.abs(g - ref).max()) / scale
        print(f"  copy {c}: rel error {err:.2e}", flush=True)
        assert np.isfinite(g).all() and err < 1e-4, (c, err)
