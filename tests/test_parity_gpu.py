"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: max-abs 1e-4 for the fp32 path and 3e-2 for the bf16 path per
output over valid rows; masked rows must be bit-exact +0.0. Inputs are the
seeded synthetic workloads; for L >= 2048 the oracle checks a fixed sample
of query rows (each query row is independent), including every tile edge.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import ipa_forward as oracle_forward
from workloads import WORKLOADS, make_inputs, round_to_bf16, stress_pair

from ipa_gpu_util import (assert_masked_positive_zero, compare, run_gpu, to_device)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 3e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(w, device, tol, seed=None, rows=None, stress=False):
    inp = make_inputs(w, seed=seed)
    if stress:
        inp = stress_pair(inp)
    _say(f"case {w.name} B={w.B} L={w.L} H={w.H} Cz={w.Cz} {w.dtype} seed={seed} stress={stress}")
    gpu = run_gpu(to_device(inp, device))
    ref = oracle_forward(inp, rows=rows)
    valid = inp["mask"].astype(bool)
    errs = compare(gpu, ref, tol, valid_rows=valid, rows=rows)
    if w.ragged is not None:
        assert_masked_positive_zero(gpu, inp["mask"])
    _say(f"  errors {errs}")
    return inp, gpu, ref, errs


def _edge_rows(L, n_random=96, seed=0):
    edges = set()
    for t in range(0, L, 64):
        edges.update({t, t + 1, t + 31, t + 32, t + 63})
    edges = {r for r in edges if r < L} | {L - 1}
    rng = np.random.default_rng(seed)
    extra = rng.choice(L, size=min(L, n_random), replace=False)
    return np.array(sorted(edges | set(extra.tolist())))


def test_tiny_fp32(device):
    _check(WORKLOADS["tiny_fp32"], device, TOL_F32)


@pytest.mark.parametrize("L", [1, 37, 200])
def test_fp32_ragged_tail(device, L):
    _check(WORKLOADS["tiny_fp32"].with_(L=L, H=3), device, TOL_F32, seed=L)


def test_fp32_odd_dims(device):
    w = WORKLOADS["tiny_fp32"].with_(L=150, H=2, C=12, Pqk=3, Pv=5, R=1, Cz=24)
    _check(w, device, TOL_F32, seed=3)


def test_single_chain_bf16(device):
    _check(WORKLOADS["single_chain"], device, TOL_BF16)


def test_single_chain_bf16_pair_stress(device):
    """Unit-variance pair factors make pair-path errors visible: the pair bias
    reaches several logits and the pair output is O(1)."""
    w = WORKLOADS["single_chain"].with_(L=256, H=4)
    inp, gpu, ref, errs = _check(w, device, 1.0, stress=True)
    for k in errs:
        rms = float(np.sqrt(np.mean(ref[k] ** 2)))
        assert errs[k] <= 3e-2 * max(rms, 1.0), (k, errs[k], rms)


def test_tiny_fp32_pair_stress(device):
    """fp32 path with unit-variance pair factors: every channel at 1e-4 of
    max(1, RMS), so the pair bias / pair output logic shared by both paths is
    checked without bf16 rounding."""
    w = WORKLOADS["tiny_fp32"].with_(L=150, H=4)
    inp, gpu, ref, errs = _check(w, device, 1.0, stress=True)
    for k in errs:
        rms = float(np.sqrt(np.mean(ref[k] ** 2)))
        assert errs[k] <= TOL_F32 * max(rms, 1.0), (k, errs[k], rms)


@pytest.mark.parametrize("L", [70, 200, 333])
def test_bf16_ragged_tail(device, L):
    _check(WORKLOADS["single_chain"].with_(L=L, H=3), device, TOL_BF16, seed=L)


def test_bf16_odd_dims(device):
    w = WORKLOADS["single_chain"].with_(L=190, H=2, C=12, Pqk=5, Pv=5, R=3, Cz=40)
    _check(w, device, TOL_BF16, seed=4)


@pytest.mark.parametrize("Cz,R", [(32, 3), (96, 2)])
def test_bf16_pair_widths(device, Cz, R):
    """Pair widths whose rank components are summed in registers (Cz a
    multiple of 32) other than the default 128, with several ranks."""
    w = WORKLOADS["single_chain"].with_(L=230, H=3, Cz=Cz, R=R)
    _check(w, device, TOL_BF16, seed=Cz)


@pytest.mark.parametrize("Cz,R", [(32, 1), (64, 1), (8, 1), (32, 2), (40, 1)])
def test_bf16_narrowest_rows(device, Cz, R):
    """R Cz <= 64: lifted rows of 128 columns, the narrowest the kernel
    runs (its value phase has the fewest product steps to schedule its
    side work into)."""
    w = WORKLOADS["single_chain"].with_(L=200, H=2, Cz=Cz, R=R)
    _check(w, device, TOL_BF16, seed=Cz + R)


def test_fp32_pair_width_32(device):
    w = WORKLOADS["tiny_fp32"].with_(L=140, H=2, Cz=32, R=2)
    _check(w, device, TOL_F32, seed=32)


def test_ragged_batch(device):
    w = WORKLOADS["ragged_batch"]
    inp = make_inputs(w)
    dev = to_device(inp, device)
    before = {k: v.clone() for k, v in dev.items() if isinstance(v, torch.Tensor)}
    gpu = run_gpu(dev)
    for k, v in before.items():
        assert torch.equal(v, dev[k]), f"input {k} was modified"
    ref = oracle_forward(inp)
    errs = compare(gpu, ref, TOL_BF16, valid_rows=inp["mask"].astype(bool))
    assert_masked_positive_zero(gpu, inp["mask"])
    _say(f"ragged batch errors {errs}")


def test_long_chain_2048_sampled(device):
    w = WORKLOADS["long_chain_2048"]
    _check(w, device, TOL_BF16, rows=_edge_rows(w.L))


@pytest.mark.parametrize("name", ["long_chain_4096", "very_long_8192", "very_long_16384"])
def test_long_sampled(device, name):
    w = WORKLOADS[name]
    _check(w, device, TOL_BF16, rows=_edge_rows(w.L, n_random=24)[::4])


def test_max_length_sampled(device):
    """L = 65536, the longest chain the envelope admits (1024 key blocks of
    64 residues, the most the attention kernel's per-block tables hold),
    with two heads; tile and block edges at the start and end of the chain
    and random rows compared with the oracle."""
    w = WORKLOADS["very_long_16384"].with_(L=65536, H=2)
    rows = _edge_rows(w.L, n_random=16, seed=5)
    rows = np.unique(np.concatenate([rows[:12], rows[-12:], rows[::len(rows) // 16]]))
    _check(w, device, TOL_BF16, rows=rows)


def test_determinism_and_noncontiguous(device):
    w = WORKLOADS["single_chain"].with_(L=300, H=4)
    inp = make_inputs(w, seed=21)
    dev = to_device(inp, device)
    a = run_gpu(dev)
    b = run_gpu(dev)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    # the same values through non-contiguous views
    nc = dict(dev)
    for k in ("q", "k", "v", "z1", "z2", "q_pts", "v_pts"):
        t = dev[k]
        big = torch.zeros((2,) + tuple(t.shape), dtype=t.dtype, device=t.device)
        big[1] = t
        view = big.transpose(0, 1)[:, 1]
        assert not view.is_contiguous() or view.data_ptr() != t.data_ptr()
        nc[k] = view
    c = run_gpu(nc)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), c[k].view(np.uint32)), k


def test_se3_invariance_gpu(device):
    w = WORKLOADS["tiny_fp32"].with_(L=128, H=4)
    inp = make_inputs(w, seed=5)
    base = run_gpu(to_device(inp, device))
    rng = np.random.default_rng(3)
    u = rng.standard_normal(4)
    u /= np.linalg.norm(u)
    a0, x, y, z = u
    Rg = np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - a0 * z), 2 * (x * z + a0 * y)],
                   [2 * (x * y + a0 * z), 1 - 2 * (x * x + z * z), 2 * (y * z - a0 * x)],
                   [2 * (x * z - a0 * y), 2 * (y * z + a0 * x), 1 - 2 * (x * x + y * y)]])
    moved = dict(inp)
    moved["rot"] = np.einsum("xy,blyz->blxz", Rg, inp["rot"].astype(np.float64)).astype(np.float32)
    moved["trans"] = (np.einsum("xy,bly->blx", Rg, inp["trans"].astype(np.float64))
                      + rng.normal(0, 100.0, 3)).astype(np.float32)
    out = run_gpu(to_device(moved, device))
    for k in base:
        np.testing.assert_allclose(out[k], base[k], rtol=0, atol=TOL_F32, err_msg=k)


def test_binding_errors(device):
    from geometric_invariant_attention_amd import IPAForward
    w = WORKLOADS["tiny_fp32"].with_(L=16, H=2)
    dev = to_device(make_inputs(w), device)
    plan = IPAForward(1, 16, 2, 16, 4, 8, 2, 16, dtype=torch.float32, device=device)
    args = {k: dev[k] for k in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans",
                                "z1", "z2", "w_b", "gamma")}
    with pytest.raises(TypeError):
        plan(**dict(args, q=args["q"].to(torch.bfloat16)))
    with pytest.raises(ValueError):
        plan(**dict(args, v=args["v"][:, :8]))
    with pytest.raises(ValueError):
        plan(**dict(args, z1=args["z1"].cpu()))


@pytest.mark.parametrize("L", [1, 7, 33])
def test_bf16_short_chains(device, L):
    """bf16 storage below one 64-residue block: a single partial key tile,
    query rows past L in the only query block."""
    _check(WORKLOADS["single_chain"].with_(L=L, H=3), device, TOL_BF16, seed=L)


def _pair_range_inputs(seed, big):
    """Pair factors at the ends of fp16's range on the bf16 path (the pair
    columns of Q.K^T are fp16 products). One rank-0 channel c0 of z2 is set
    to +-6e4 (near the largest finite fp16, 65504) with z1 there at 3e-4,
    or (big=False) to +-1.5e-5 (an fp16 subnormal, below 2^-14) with z1 there
    at 5e4 and W_b[c0, :] = 1, so the query operand w_L log2(e) W_b z1 is
    about 4.2e4. Either way that channel moves logits by several units and
    the pair output by O(1)."""
    w = WORKLOADS["single_chain"].with_(L=300, H=4, Cz=32, R=2)
    inp = make_inputs(w, seed=seed)
    rng = np.random.default_rng(seed + 1)
    L, Cz = w.L, w.Cz
    sign = np.where(rng.random((1, L)) < 0.5, -1.0, 1.0)
    c0 = 5
    z1, z2, wb = inp["z1"].copy(), inp["z2"].copy(), inp["w_b"].copy()
    if big:
        z2[:, :, 0, c0] = sign * 6.0e4 * rng.uniform(0.9, 1.0, size=(1, L))
        z1[:, :, 0, c0] = 3.0e-4 * rng.uniform(0.5, 1.0, size=(1, L))
    else:
        z2[:, :, 0, c0] = sign * 1.5e-5 * rng.uniform(0.5, 1.0, size=(1, L))
        z1[:, :, 0, c0] = 5.0e4 * rng.uniform(0.9, 1.0, size=(1, L))
        wb[c0, :] = 1.0
    inp["z1"] = round_to_bf16(z1)
    inp["z2"] = round_to_bf16(z2)
    inp["w_b"] = wb.astype(np.float32)
    return w, inp


@pytest.mark.parametrize("big", [True, False])
def test_bf16_pair_fp16_range_ends(device, big):
    """Inside the documented fp16 range of the pair columns the logits keep
    their value at both ends: near +-65504 and below 2^-14. Errors are
    taken relative to max(1, RMS) per output, as in the pair-stress test."""
    w, inp = _pair_range_inputs(17 if big else 18, big)
    _say(f"case pair fp16 range big={big} L={w.L} H={w.H} Cz={w.Cz}")
    gpu = run_gpu(to_device(inp, device))
    ref = oracle_forward(inp)
    for k in ref:
        assert np.all(np.isfinite(gpu[k])), k
        err = float(np.abs(gpu[k].astype(np.float64) - ref[k]).max())
        rms = float(np.sqrt(np.mean(ref[k] ** 2)))
        _say(f"  {k}: max-abs {err:.3e}, rms {rms:.3e}")
        assert err <= TOL_BF16 * max(rms, 1.0), (k, err, rms)


def test_side_stream_binding(device):
    """Kernels launched on a stream other than the current one, with inputs
    that need contiguous copies: the copies are ordered before the kernels
    and the result equals the current-stream call bit for bit."""
    from geometric_invariant_attention_amd import IPAForward
    w = WORKLOADS["single_chain"].with_(L=256, H=4)
    inp = make_inputs(w, seed=31)
    dev = to_device(inp, device)
    base = run_gpu(dev)
    names = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "w_b", "gamma")
    nc = {}
    for k in names:
        t = dev[k]
        big = torch.zeros((2,) + tuple(t.shape), dtype=t.dtype, device=t.device)
        big[1] = t
        nc[k] = big.transpose(0, 1)[:, 1]
    plan = IPAForward(**w.dims(), dtype=torch.bfloat16, device=device)
    side = torch.cuda.Stream(device)
    out = plan(**nc, w_L=dev["w_L"], w_C=dev["w_C"], stream=side)
    side.synchronize()
    for k in base:
        assert np.array_equal(base[k].view(np.uint32), out[k].cpu().numpy().view(np.uint32)), k
