"""The pair part of the attention's running-max seed, as the lift writes it.

For every residue i, head h and 64-wide pair panel P the lift stores
sum_u sat(w_L log2(e) W_b[u mod Cz, h] z1[i, u]) sat(z2[i, u]) over the
panel's features u < R Cz (sat: clamp to fp16's finite range), zero for
masked residues: the pair part of the logit of query i with its own key as
the attention's fp16 products take it. This test reads that per-panel array
back from the workspace (its offset follows the library's workspace layout,
which the test recomputes) and checks it against the same sum in float64,
in the regimes of the kernel: matrix-core products (no operand near the
fp16 limit), several chunks of 16 heads, the clamped path (z1 scaled by
2^17 so that w_L log2(e) W_b z1 exceeds 65504) and a scattered mask. The
tolerance covers fp16 rounding of the products' operands with float32
accumulation.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _align256(x):
    return (x + 255) & ~255


def _pdiag_offset(B, L, H, R, Cz, es=2):
    """Byte offset of the [B][H][Lp] float4 per-panel seed array."""
    Lp = (L + 127) // 128 * 128
    nJ = Lp // 64
    PW = (R * Cz + 63) // 64 * 64
    sizes = [B * H * Lp * 64 * es, B * H * Lp * 64 * es, B * nJ * PW * 64 * es, B * H * nJ * 64 * 64 * es,
             B * nJ * PW * 64 * es, B * H * Lp * 16, B * H * Lp * 16, B * nJ * 16]
    off = 0
    for s in sizes:
        off = _align256(off + s)
    return off, Lp, PW // 64


def _expected(inp, Lp, npanel):
    d = inp["dims"]
    B, L, H, R, Cz = d["B"], d["L"], d["H"], d["R"], d["Cz"]
    z1 = inp["z1"].astype(np.float64).reshape(B, L, R * Cz)
    z2 = inp["z2"].astype(np.float64).reshape(B, L, R * Cz)
    wb = inp["w_b"].astype(np.float64)                          # [Cz, H]
    wsc = float(np.float32(inp["w_L"]) * np.float32(LOG2E))
    u = np.arange(R * Cz)
    W = wsc * wb[u % Cz]                                         # [R Cz, H]
    sat = lambda x: np.clip(x, -65504.0, 65504.0)
    out = np.zeros((B, H, Lp, 4))
    scale = np.zeros((B, H, Lp, 4))
    for P in range(npanel):
        sl = slice(64 * P, min(64 * P + 64, R * Cz))
        q = sat(z1[:, :, None, sl] * W[None, None, sl].transpose(0, 1, 3, 2))   # [B, L, H, u]
        k = sat(z2[:, :, None, sl])
        out[:, :, :L, P] = np.einsum("blhu,blhu->bhl", q, np.broadcast_to(k, q.shape))
        scale[:, :, :L, P] = np.einsum("blhu,blhu->bhl", np.abs(q), np.abs(np.broadcast_to(k, q.shape)))
    m = inp["mask"].astype(bool)
    out[:, :, :L][~np.broadcast_to(m[:, None, :], (B, H, L))] = 0.0
    return out, scale


def _run(inp):
    from geometric_invariant_attention_amd import _binding as Bd
    lib = Bd.load_library()
    d = inp["dims"]
    dev = torch.device("cuda", 0)
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(torch.bfloat16).to(dev)
         for k in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2")}
    for k in ("rot", "trans", "w_b", "gamma"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev)
    mask = torch.from_numpy(inp["mask"]).to(dev) if inp.get("has_mask") else None
    dims = Bd.IpaDims(**d)
    wsb = lib.ipa_workspace_bytes(ctypes.byref(dims), 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    outs = [torch.empty(d["B"], d["L"], d["H"], n, device=dev) for n in (d["C"], 3 * d["Pv"], d["Pv"], d["Cz"])]
    st = torch.cuda.current_stream(dev)
    raw = (ctypes.byref(dims), 1, *(t[n].data_ptr() for n in ("q", "k", "v", "q_pts", "k_pts", "v_pts",
                                                               "rot", "trans", "z1", "z2", "w_b", "gamma")),
           0 if mask is None else mask.data_ptr(), ctypes.c_float(inp["w_L"]), ctypes.c_float(inp["w_C"]),
           *(o.data_ptr() for o in outs), ws.data_ptr(), ctypes.c_size_t(wsb), ctypes.c_void_p(st.cuda_stream))
    assert lib.ipa_lift(*raw) == 0
    torch.cuda.synchronize()
    return ws.cpu().numpy()


@pytest.mark.parametrize("case", ["plain", "two_chunks", "clamped", "masked"])
def test_lift_pair_seed(device, case):
    w = WORKLOADS["long_chain_2048"].with_(L=300, H=5)
    if case == "two_chunks":
        w = w.with_(L=200, H=20)
    if case == "masked":
        w = WORKLOADS["single_chain"].with_(B=3, L=333, H=3, mask="scatter")
    inp = make_inputs(w, seed=7)
    if case == "clamped":
        inp = dict(inp)
        inp["z1"] = (inp["z1"].astype(np.float32) * np.float32(131072.0)).astype(inp["z1"].dtype)
    d = inp["dims"]
    print(f"[seed] {case}: B={d['B']} L={d['L']} H={d['H']} R Cz={d['R'] * d['Cz']}", flush=True)
    off, Lp, npanel = _pdiag_offset(d["B"], d["L"], d["H"], d["R"], d["Cz"])
    ws = _run(inp)
    got = ws[off:off + d["B"] * d["H"] * Lp * 16].view(np.float32).reshape(d["B"], d["H"], Lp, 4)
    exp, scale = _expected(inp, Lp, npanel)
    g = got[:, :, :d["L"], :npanel].astype(np.float64)
    e = exp[:, :, :d["L"], :npanel]
    s = scale[:, :, :d["L"], :npanel]
    if case == "clamped":
        wsc = inp["w_L"] * LOG2E
        assert np.abs(inp["z1"].astype(np.float64)).max() * np.abs(inp["w_b"]).max() * wsc > 65504.0
    err = np.abs(g - e) / (s + 1e-30)
    print(f"  max relative error {err.max():.2e} (worst at {np.unravel_index(np.argmax(err), err.shape)})", flush=True)
    assert np.all(np.isfinite(g))
    assert np.all(np.abs(g - e) <= 2e-3 * s + 1e-6)
