"""GPU parity of the direction-and-distance attention against the fp64
oracle, through the C ABI (ipa_dirdist_forward).

Tolerance: the kernels compute in float32 with the square root and the
base-2 exponential of the hardware (about 1 ulp each). At these shapes the
logits are O(10^2) at most and each output a convex combination of O(1)
values, so float32 rounding stays near 1e-5; 1e-4 absolute on vectors and
attention, and 1e-4 relative to the output's scale on the readout
(a 3HM-term sum), leave room without hiding a wrong term.
"""

import numpy as np
import pytest
import torch

from oracle import dirdist_attention
from workloads import DIRDIST_WORKLOADS, make_dirdist_inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4
ARGS = ("rot", "trans", "q_direction", "k_direction", "q_point", "k_point", "values",
        "direction_scale", "distance_scale", "output_weight", "output_bias")


def _gpu(inp, device, attention=True, pair_mask="as_is"):
    from geometric_invariant_attention_amd import DirDistForward
    d = inp["dims"]
    t = {k: (torch.from_numpy(inp[k]).to(device) if inp[k] is not None else None) for k in ARGS}
    fm = torch.from_numpy(inp["frame_mask"]).to(device)
    pm = inp["pair_mask"] if isinstance(pair_mask, str) else pair_mask
    pm = torch.from_numpy(np.ascontiguousarray(pm)).to(device) if pm is not None else None
    plan = DirDistForward(d["B"], d["N"], d["H"], d["M"], d["Cout"], device=device, attention=attention)
    out = plan(*(t[k] for k in ARGS), frame_mask=fm, pair_mask=pm)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().copy() for k, v in out.items()}


def _oracle(inp):
    return dirdist_attention(**{k: inp[k] for k in ARGS}, frame_mask=inp["frame_mask"],
                             pair_mask=inp["pair_mask"])


def _check(inp, gpu, ref, attention=True):
    assert np.isfinite(gpu["vectors"]).all() and np.isfinite(gpu["output"]).all()
    ev = float(np.abs(gpu["vectors"] - ref["vectors"]).max())
    scale = max(1.0, float(np.abs(ref["output"]).max()))
    eo = float(np.abs(gpu["output"] - ref["output"]).max()) / scale
    errs = {"vectors": ev, "output": eo}
    if attention:
        errs["attention"] = float(np.abs(gpu["attention"] - ref["attention"]).max())
    assert max(errs.values()) < TOL, errs
    # exact positive zeros wherever the oracle's are exactly zero by rule
    for k in gpu:
        z = ref[k] == 0
        if k == "attention" or k == "output":
            assert np.all(gpu[k][z] == 0) and not np.signbit(gpu[k][z]).any(), k
    return errs


def _run(w, device, seed=None, attention=True):
    print(f"[dirdist] {w.name} dims={w.dims()} pm={w.pair_mask} ragged={w.ragged} seed={seed}", flush=True)
    inp = make_dirdist_inputs(w, seed=seed)
    gpu = _gpu(inp, device, attention=attention)
    ref = _oracle(inp)
    return inp, gpu, ref, _check(inp, gpu, ref, attention)


def test_tiny_full_pair_mask(device):
    _run(DIRDIST_WORKLOADS["dd_tiny_fp32"], device)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_value_count(device, M):
    _run(DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(N=45, H=2, M=M, Cout=7), device, seed=M)


@pytest.mark.parametrize("N", [1, 2, 7, 8, 9, 63, 64, 65, 300])
def test_ragged_lengths(device, N):
    w = DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(N=N, B=1, H=3, M=4, Cout=33, ragged=None,
                                                pair_mask=None)
    _run(w, device, seed=N)


@pytest.mark.parametrize("kind", ["shared", "per_head", "full"])
def test_pair_mask_broadcast_kinds(device, kind):
    _run(DIRDIST_WORKLOADS["dd_ragged"].with_(B=3, N=70, ragged=(30, 70), pair_mask=kind), device)


def test_ragged_batch(device):
    inp, gpu, ref, _ = _run(DIRDIST_WORKLOADS["dd_ragged"], device)
    pad = inp["frame_mask"] == 0
    assert np.all(gpu["output"][pad] == 0) and np.all(gpu["vectors"][pad] == 0)


def test_no_bias_and_no_attention(device):
    w = DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(bias=False)
    _run(w, device, attention=False)


def test_empty_heads_and_rows(device):
    """A query whose every head is masked gets a zero output despite the bias;
    a query with one empty head keeps its output."""
    w = DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(B=1, N=40, H=3, ragged=None, pair_mask=None)
    inp = make_dirdist_inputs(w, seed=11)
    pm = np.ones((1, 3, 40, 40), np.uint8)
    pm[0, :, 5, :] = 0
    pm[0, 1, 6, :] = 0
    inp["pair_mask"] = pm
    gpu = _gpu(inp, device)
    ref = _oracle(inp)
    _check(inp, gpu, ref)
    assert np.all(gpu["output"][0, 5] == 0) and np.abs(gpu["output"][0, 6]).max() > 0


def test_chain_512(device):
    _run(DIRDIST_WORKLOADS["dd_chain_512"], device, attention=False)


def test_chain_2048_sampled_rows(device):
    """Full size, as measured: the oracle checks a sample of query rows (each
    row is independent) and the attention rows of those queries."""
    w = DIRDIST_WORKLOADS["dd_chain_2048"]
    print(f"[dirdist] {w.name} dims={w.dims()} sampled", flush=True)
    inp = make_dirdist_inputs(w)
    gpu = _gpu(inp, device, attention=True)
    rows = np.sort(np.random.default_rng(0).choice(w.N, 48, replace=False))
    ref = dirdist_attention(**{k: inp[k] for k in ARGS}, frame_mask=inp["frame_mask"], rows=rows)
    ev = np.abs(gpu["vectors"][:, rows] - ref["vectors"]).max()
    ea = np.abs(gpu["attention"][:, :, rows] - ref["attention"]).max()
    eo = np.abs(gpu["output"][:, rows] - ref["output"]).max() / max(1.0, np.abs(ref["output"]).max())
    assert max(ev, ea, eo) < TOL, (ev, ea, eo)
    # every attention row of a valid query sums to one
    s = gpu["attention"].sum(-1)
    assert np.abs(s - 1).max() < 1e-4


def test_repeat_calls_are_bitwise_identical(device):
    inp = make_dirdist_inputs(DIRDIST_WORKLOADS["dd_ragged"])
    a = _gpu(inp, device)
    b = _gpu(inp, device)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_inputs_are_not_modified(device):
    from geometric_invariant_attention_amd import geometric_reasoning_attention
    inp = make_dirdist_inputs(DIRDIST_WORKLOADS["dd_tiny_fp32"])
    t = {k: torch.from_numpy(inp[k]).to(device) for k in ARGS}
    before = {k: v.clone() for k, v in t.items()}
    fm = torch.from_numpy(inp["frame_mask"]).to(device)
    pm = torch.from_numpy(inp["pair_mask"]).to(device).bool()
    # non-contiguous views are accepted
    t["output_weight"] = t["output_weight"].t().contiguous().t()
    out = geometric_reasoning_attention(*(t[k] for k in ARGS), frame_mask=fm, pair_mask=pm)
    torch.cuda.synchronize()
    for k in before:
        assert torch.equal(before[k], t[k]), k
    ref = _oracle(inp)
    assert np.abs(out["vectors"].cpu().numpy() - ref["vectors"]).max() < TOL



def test_wide_value_rows(device):
    """24 heads of 8 value vectors (576 flattened values per query row):
    the readout's reduction spans several of its load batches."""
    w = DIRDIST_WORKLOADS["dd_tiny_fp32"].with_(B=2, N=70, H=24, M=8, Cout=40, ragged=(30, 70),
                                                pair_mask="per_head")
    _run(w, device, seed=5)
