"""ipa_forward_noalloc (the forward whose workspace is the library's static
device array) against ipa_forward (caller workspace) through the C ABI.

Two calls in a row on the static array, the second on a smaller problem
with a scattered mask, so that it runs over what the first left behind;
then the first problem again. Each result must equal ipa_forward's
bit for bit (the same kernels run on the same inputs, and the forward is
deterministic), and the masked one is also checked against the fp64 oracle
at the bf16 tolerance with masked rows +0.0. Dims that need more than the
static array are refused before anything is enqueued.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import ipa_forward as oracle_forward
from workloads import WORKLOADS, make_inputs

from ipa_gpu_util import FEATS, FRAMES, OUTS, assert_masked_positive_zero, compare, to_device

pytestmark = pytest.mark.gpu


def _plan_and_raw(w, device, seed):
    from geometric_invariant_attention_amd import IPAForward
    inp = make_inputs(w, seed=seed)
    t = to_device(inp, device)
    plan = IPAForward(**w.dims(), dtype=torch.bfloat16, device=device)
    raw = plan.bind(**{k: t[k] for k in FEATS + FRAMES}, mask=t["mask"], w_L=t["w_L"], w_C=t["w_C"])
    return inp, plan, raw


def _outputs(plan) -> dict:
    torch.cuda.synchronize()
    return {k: plan.out[k].detach().cpu().numpy().copy() for k in OUTS}


def _fill(plan, value):
    for o in plan.out.values():
        o.fill_(value)


def _same_bits(a: dict, b: dict, what: str):
    for k in OUTS:
        assert a[k].shape == b[k].shape
        diff = np.flatnonzero(a[k].view(np.uint32) != b[k].view(np.uint32))
        assert diff.size == 0, f"{what}: {k} differs at {diff.size} elements (first {diff[:5]})"


def test_noalloc_matches_forward_two_calls(device):
    big = WORKLOADS["long_chain_2048"]
    small = WORKLOADS["single_chain"].with_(B=3, L=700, H=5, mask="scatter")
    cases = []
    for w, seed in ((big, 0), (small, 11)):
        print(f"[noalloc] {w.name} B={w.B} L={w.L} H={w.H} mask={w.mask}", flush=True)
        inp, plan, raw = _plan_and_raw(w, device, seed)
        assert plan.ws_bytes <= 64 << 20
        plan.forward_raw(raw)
        ref = _outputs(plan)
        cases.append((w, inp, plan, raw, ref))
    # the static array: big, then small over its leftovers, then big again
    for idx in (0, 1, 0):
        w, inp, plan, raw, ref = cases[idx]
        print(f"[noalloc] static workspace call on {w.name} L={w.L}", flush=True)
        _fill(plan, float("nan"))
        plan.forward_noalloc_raw(raw)
        got = _outputs(plan)
        _same_bits(got, ref, f"{w.name} L={w.L}")
        if w.mask == "scatter":
            errs = compare(got, oracle_forward(inp), 3e-2, valid_rows=inp["mask"].astype(bool))
            assert_masked_positive_zero(got, inp["mask"])
            print(f"  oracle errors {errs}", flush=True)


def test_noalloc_refuses_oversize_dims(device):
    from geometric_invariant_attention_amd import load_library
    from geometric_invariant_attention_amd import _binding as bd
    lib = load_library()
    d = bd.IpaDims(B=1, L=16384, H=8, C=16, Pqk=4, Pv=8, R=2, Cz=128)
    assert lib.ipa_workspace_bytes(ctypes.byref(d), bd.IPA_BF16) > 64 << 20
    ptr = 0x100000
    rc = lib.ipa_forward_noalloc(ctypes.byref(d), bd.IPA_BF16, *([ptr] * 12), None, ctypes.c_float(0.5),
                                 ctypes.c_float(0.3), *([ptr] * 4), None)
    assert rc == -9, bd.status_string(rc)
    assert "IPA_NOALLOC_WORKSPACE_BYTES" in bd.status_string(rc)
