"""ctypes binding of the C ABI in include/ipa.h.

Argument marshalling only: every step of the IPA forward runs in the HIP
library. PyTorch provides device memory and the current stream. If the
library is missing this module raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = Path(os.environ.get("IPA_MI355_LIB", _PKG / "libipa_mi355.so"))

IPA_F32 = 0
IPA_BF16 = 1

STATUS = {
    0: "IPA_OK", -1: "IPA_ERR_NULL", -2: "IPA_ERR_DIMS", -3: "IPA_ERR_DTYPE",
    -4: "IPA_ERR_WORKSPACE", -5: "IPA_ERR_ALIGN", -6: "IPA_ERR_UNSUPPORTED",
    -7: "IPA_ERR_HIP", -8: "IPA_ERR_ARG", -9: "IPA_ERR_LIMIT",
}


class IpaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "H", "C", "Pqk", "Pv", "R", "Cz")]


class IpaMeetDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "H", "C")]


class IpaDirDistDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "N", "H", "M", "Cout")]


class IPAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str | os.PathLike | None = None) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(
            f"IPA HIP library not found at {p}; build it with "
            "`python -m geometric_invariant_attention_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    lib.ipa_workspace_bytes.argtypes = [ctypes.POINTER(IpaDims), i32]
    lib.ipa_workspace_bytes.restype = sz
    for fn in (lib.ipa_forward, lib.ipa_lift, lib.ipa_attend):
        fn.argtypes = [ctypes.POINTER(IpaDims), i32] + [vp] * 13 + [f32, f32] + [vp] * 5 + [sz, vp]
        fn.restype = i32
    lib.ipa_forward_noalloc.argtypes = [ctypes.POINTER(IpaDims), i32] + [vp] * 13 + [f32, f32] + [vp] * 4 + [vp]
    lib.ipa_forward_noalloc.restype = i32
    lib.ipa_frames_from_atoms.argtypes = [i32, i32] + [vp] * 5 + [vp]
    lib.ipa_frames_from_atoms.restype = i32
    lib.ipa_meet_workspace_bytes.argtypes = [ctypes.POINTER(IpaMeetDims), i32]
    lib.ipa_meet_workspace_bytes.restype = sz
    lib.ipa_meet_forward.argtypes = [ctypes.POINTER(IpaMeetDims), i32] + [vp] * 9 + [sz, vp]
    lib.ipa_meet_forward.restype = i32
    lib.ipa_dirdist_workspace_bytes.argtypes = [ctypes.POINTER(IpaDirDistDims)]
    lib.ipa_dirdist_workspace_bytes.restype = sz
    lib.ipa_dirdist_forward.argtypes = [ctypes.POINTER(IpaDirDistDims)] + [vp] * 18 + [sz, vp]
    lib.ipa_dirdist_forward.restype = i32
    lib.ipa_backward_workspace_bytes.argtypes = [ctypes.POINTER(IpaDims)]
    lib.ipa_backward_workspace_bytes.restype = sz
    lib.ipa_backward.argtypes = [ctypes.POINTER(IpaDims)] + [vp] * 13 + [f32, f32] + [vp] * 20 + [sz, vp]
    lib.ipa_backward.restype = i32
    lib.ipa_backward_flash_workspace_bytes.argtypes = [ctypes.POINTER(IpaDims)]
    lib.ipa_backward_flash_workspace_bytes.restype = sz
    lib.ipa_backward_flash.argtypes = [ctypes.POINTER(IpaDims), i32] + [vp] * 13 + [f32, f32] + [vp] * 20 + [sz, vp]
    lib.ipa_backward_flash.restype = i32
    lib.ipa_layer_workspace_bytes.argtypes = [ctypes.POINTER(IpaDims), i32, i32]
    lib.ipa_layer_workspace_bytes.restype = sz
    lib.ipa_layer_forward.argtypes = [ctypes.POINTER(IpaDims), i32, i32] + [vp] * 8 + [f32, f32] + [vp] * 4 + [sz, vp]
    lib.ipa_layer_forward.restype = i32
    lib.ipa_status_string.argtypes = [i32]
    lib.ipa_status_string.restype = ctypes.c_char_p
    lib.ipa_version.argtypes = []
    lib.ipa_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ipa_status_string(status).decode()


def make_dims(B, L, H, C, Pqk, Pv, R, Cz) -> IpaDims:
    return IpaDims(B, L, H, C, Pqk, Pv, R, Cz)


def workspace_bytes(dims: dict | IpaDims, dtype: int) -> int:
    d = dims if isinstance(dims, IpaDims) else IpaDims(**dims)
    return int(load_library().ipa_workspace_bytes(ctypes.byref(d), int(dtype)))


def default_weights(Pqk: int) -> tuple[float, float]:
    return math.sqrt(1.0 / 3.0), math.sqrt(2.0 / (9.0 * Pqk))


def _dev_ptr(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.data_ptr()


def _prep(t: torch.Tensor, dtype: torch.dtype, device, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous() or t.data_ptr() % 16 != 0:
        t = t.contiguous() if not t.is_contiguous() else t.clone()
    return t


def _order_on(stream, device, tensors) -> "torch.cuda.Stream":
    """Return the stream the kernels run on (the current one if ``stream``
    is None). The contiguous copies and mask conversions made while binding
    run on the current stream; when the kernels go to another stream, that
    stream first waits for the current one, and every tensor the kernels
    touch is recorded on it so that the caching allocator does not hand its
    memory out again before they finish."""
    cur = torch.cuda.current_stream(device)
    if stream is None or stream == cur:
        return cur
    stream.wait_stream(cur)
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(stream)
    return stream


class IPAForward:
    """Reusable forward plan: validated shapes, preallocated workspace and
    outputs on one device. ``__call__`` enqueues one forward on the current
    stream and returns the output dict (the same tensors on every call)."""

    def __init__(self, B, L, H, C, Pqk, Pv, R, Cz, dtype=torch.bfloat16, device=None):
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be torch.bfloat16 or torch.float32")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = IpaDims(B, L, H, C, Pqk, Pv, R, Cz)
        self.shape = dict(B=B, L=L, H=H, C=C, Pqk=Pqk, Pv=Pv, R=R, Cz=Cz)
        self.dtype = dtype
        self.code = IPA_BF16 if dtype == torch.bfloat16 else IPA_F32
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_workspace_bytes(ctypes.byref(self.dims), self.code))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape} for {dtype}")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.out = {
            "s": torch.empty(B, L, H, C, **f32),
            "pts": torch.empty(B, L, H, Pv, 3, **f32),
            "pts_norm": torch.empty(B, L, H, Pv, **f32),
            "pair": torch.empty(B, L, H, Cz, **f32),
        }

    def bind(self, q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma,
             mask=None, w_L=None, w_C=None, stream=None) -> tuple:
        """Validate the tensors once and return the raw argument tuple of the
        C entry points (tensors that needed a contiguous copy are kept alive
        in ``self.bound``)."""
        s = self.shape
        B, L, H, C, Pqk, Pv, R, Cz = (s[n] for n in ("B", "L", "H", "C", "Pqk", "Pv", "R", "Cz"))
        dev, dt = self.device, self.dtype
        expect = {
            "q": (B, L, H, C), "k": (B, L, H, C), "v": (B, L, H, C),
            "q_pts": (B, L, H, Pqk, 3), "k_pts": (B, L, H, Pqk, 3), "v_pts": (B, L, H, Pv, 3),
            "z1": (B, L, R, Cz), "z2": (B, L, R, Cz),
            "rot": (B, L, 3, 3), "trans": (B, L, 3), "w_b": (Cz, H), "gamma": (H,),
        }
        args = dict(q=q, k=k, v=v, q_pts=q_pts, k_pts=k_pts, v_pts=v_pts, z1=z1, z2=z2,
                    rot=rot, trans=trans, w_b=w_b, gamma=gamma)
        for name, shp in expect.items():
            t = args[name]
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
            want = dt if name in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2") else torch.float32
            args[name] = _prep(t, want, dev, name)
        m = None
        if mask is not None:
            if tuple(mask.shape) != (B, L):
                raise ValueError(f"mask has shape {tuple(mask.shape)}, expected {(B, L)}")
            if mask.device != dev:
                raise ValueError(f"mask is on {mask.device}, expected {dev}")
            m = mask.to(torch.uint8) if mask.dtype != torch.uint8 else mask
            m = m.contiguous()
        dwL, dwC = default_weights(Pqk)
        w_L = dwL if w_L is None else float(w_L)
        w_C = dwC if w_C is None else float(w_C)
        o = self.out
        stream = _order_on(stream, dev, [*args.values(), m, self.workspace, *o.values()])
        self.bound = (args, m)
        return (ctypes.byref(self.dims), self.code,
                *(_dev_ptr(args[n]) for n in ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot",
                                              "trans", "z1", "z2", "w_b", "gamma")),
                _dev_ptr(m), ctypes.c_float(w_L), ctypes.c_float(w_C),
                o["s"].data_ptr(), o["pts"].data_ptr(), o["pts_norm"].data_ptr(), o["pair"].data_ptr(),
                self.workspace.data_ptr(), ctypes.c_size_t(self.ws_bytes),
                ctypes.c_void_p(stream.cuda_stream))

    def _call(self, fn, raw: tuple) -> None:
        rc = fn(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))

    def forward_raw(self, raw: tuple) -> dict:
        self._call(self.lib.ipa_forward, raw)
        return self.out

    def forward_noalloc_raw(self, raw: tuple) -> dict:
        """ipa_forward_noalloc on the arguments of ``bind`` (the plan's own
        workspace is not passed: the library's static one is used)."""
        self._call(self.lib.ipa_forward_noalloc, raw[:-3] + raw[-1:])
        return self.out

    def lift_raw(self, raw: tuple) -> None:
        self._call(self.lib.ipa_lift, raw)

    def attend_raw(self, raw: tuple) -> dict:
        self._call(self.lib.ipa_attend, raw)
        return self.out

    def __call__(self, *args, **kw) -> dict:
        return self.forward_raw(self.bind(*args, **kw))


def ipa_forward(q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma,
                mask=None, w_L=None, w_C=None) -> dict:
    """One IPA forward on the device of ``q``; returns freshly allocated
    float32 outputs {"s", "pts", "pts_norm", "pair"}."""
    B, L, H, C = q.shape
    Pqk, Pv = q_pts.shape[3], v_pts.shape[3]
    R, Cz = z1.shape[2], z1.shape[3]
    plan = IPAForward(B, L, H, C, Pqk, Pv, R, Cz, dtype=q.dtype, device=q.device)
    out = plan(q, k, v, q_pts, k_pts, v_pts, rot, trans, z1, z2, w_b, gamma,
               mask=mask, w_L=w_L, w_C=w_C)
    return out


def frames_from_atoms(n: torch.Tensor, ca: torch.Tensor, c: torch.Tensor,
                      stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Residue frames (rot [B,L,3,3], trans [B,L,3], float32) from backbone
    atoms n, ca, c [B,L,3] float32 on one device (ipa_frames_from_atoms)."""
    if n.dim() != 3 or n.shape[-1] != 3 or ca.shape != n.shape or c.shape != n.shape:
        raise ValueError(f"atoms must share a [B,L,3] shape, got {tuple(n.shape)}, "
                         f"{tuple(ca.shape)}, {tuple(c.shape)}")
    dev = n.device
    n, ca, c = (_prep(t, torch.float32, dev, name) for t, name in ((n, "n"), (ca, "ca"), (c, "c")))
    B, L = n.shape[0], n.shape[1]
    rot = torch.empty(B, L, 3, 3, dtype=torch.float32, device=dev)
    trans = torch.empty(B, L, 3, dtype=torch.float32, device=dev)
    stream = _order_on(stream, dev, [n, ca, c, rot, trans])
    rc = load_library().ipa_frames_from_atoms(B, L, n.data_ptr(), ca.data_ptr(), c.data_ptr(),
                                              rot.data_ptr(), trans.data_ptr(),
                                              ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise IPAError(rc, status_string(rc))
    return rot, trans


def meet_workspace_bytes(B: int, L: int, H: int, C: int, dtype: int) -> int:
    d = IpaMeetDims(B, L, H, C)
    return int(load_library().ipa_meet_workspace_bytes(ctypes.byref(d), int(dtype)))


class MeetForward:
    """Reusable plan of the distance-penalised attention (ipa_meet_forward):
    validated shapes, preallocated workspace and output on one device."""

    def __init__(self, B, L, H, C, dtype=torch.bfloat16, device=None):
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be torch.bfloat16 or torch.float32")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = IpaMeetDims(B, L, H, C)
        self.shape = dict(B=B, L=L, H=H, C=C)
        self.dtype = dtype
        self.code = IPA_BF16 if dtype == torch.bfloat16 else IPA_F32
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_meet_workspace_bytes(ctypes.byref(self.dims), self.code))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape} for {dtype}")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.out = torch.empty(B, L, H, C, dtype=torch.float32, device=self.device)

    def bind(self, q, k, v, x, rho, s, mask=None, stream=None) -> tuple:
        B, L, H, C = (self.shape[n] for n in ("B", "L", "H", "C"))
        dev, dt = self.device, self.dtype
        expect = {"q": ((B, L, H, C), dt), "k": ((B, L, H, C), dt), "v": ((B, L, H, C), dt),
                  "x": ((B, L, 3), torch.float32), "rho": ((H,), torch.float32), "s": ((H,), torch.float32)}
        args = dict(q=q, k=k, v=v, x=x, rho=rho, s=s)
        for name, (shp, want) in expect.items():
            t = args[name]
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
            args[name] = _prep(t, want, dev, name)
        m = None
        if mask is not None:
            if tuple(mask.shape) != (B, L):
                raise ValueError(f"mask has shape {tuple(mask.shape)}, expected {(B, L)}")
            if mask.device != dev:
                raise ValueError(f"mask is on {mask.device}, expected {dev}")
            m = (mask.to(torch.uint8) if mask.dtype != torch.uint8 else mask).contiguous()
        stream = _order_on(stream, dev, [*args.values(), m, self.workspace, self.out])
        self.bound = (args, m)
        return (ctypes.byref(self.dims), self.code,
                *(args[n].data_ptr() for n in ("q", "k", "v", "x", "rho", "s")),
                _dev_ptr(m), self.out.data_ptr(), self.workspace.data_ptr(),
                ctypes.c_size_t(self.ws_bytes), ctypes.c_void_p(stream.cuda_stream))

    def forward_raw(self, raw: tuple) -> torch.Tensor:
        rc = self.lib.ipa_meet_forward(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))
        return self.out

    def __call__(self, *args, **kw) -> torch.Tensor:
        return self.forward_raw(self.bind(*args, **kw))


def meet_attention(q, k, v, x, rho, s, mask=None) -> torch.Tensor:
    """Distance-penalised attention on the device of ``q``: per head h,
    softmax_j(rho_h (q_i . k_j - s_h^2 |x_i - x_j|^2)) applied to v.
    Returns a freshly allocated float32 [B,L,H,C] tensor."""
    B, L, H, C = q.shape
    plan = MeetForward(B, L, H, C, dtype=q.dtype, device=q.device)
    return plan(q, k, v, x, rho, s, mask=mask)


# ---------------------------------------------------------------------------
# direction-and-distance attention (ipa_dirdist_forward)
# ---------------------------------------------------------------------------
def dirdist_workspace_bytes(B: int, N: int, H: int, M: int, Cout: int) -> int:
    d = IpaDirDistDims(B, N, H, M, Cout)
    return int(load_library().ipa_dirdist_workspace_bytes(ctypes.byref(d)))


class DirDistForward:
    """Reusable plan of the direction-and-distance attention
    (ipa_dirdist_forward): validated shapes, preallocated workspace and
    outputs on one device. Inputs may be non-contiguous (contiguous copies
    are passed on; the caller's tensors are never written)."""

    def __init__(self, B, N, H, M, Cout, device=None, attention=False):
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = IpaDirDistDims(B, N, H, M, Cout)
        self.shape = dict(B=B, N=N, H=H, M=M, Cout=Cout)
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_dirdist_workspace_bytes(ctypes.byref(self.dims)))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape}")
        dev = self.device
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.vectors = torch.empty(B, N, H, M, 3, dtype=torch.float32, device=dev)
        self.output = torch.empty(B, N, Cout, dtype=torch.float32, device=dev)
        self.attention = torch.empty(B, H, N, N, dtype=torch.float32, device=dev) if attention else None

    def bind(self, rot, trans, q_direction, k_direction, q_point, k_point, values,
             direction_scale, distance_scale, output_weight, output_bias=None,
             frame_mask=None, pair_mask=None, stream=None) -> tuple:
        B, N, H, M, Cout = (self.shape[n] for n in ("B", "N", "H", "M", "Cout"))
        dev, f32 = self.device, torch.float32
        expect = {"rot": (B, N, 3, 3), "trans": (B, N, 3), "q_direction": (B, N, H, 3),
                  "k_direction": (B, N, H, 3), "q_point": (B, N, H, 3), "k_point": (B, N, H, 3),
                  "values": (B, N, H, M, 3), "direction_scale": (H,), "distance_scale": (H,),
                  "output_weight": (3 * H * M, Cout)}
        args = dict(rot=rot, trans=trans, q_direction=q_direction, k_direction=k_direction,
                    q_point=q_point, k_point=k_point, values=values,
                    direction_scale=direction_scale, distance_scale=distance_scale,
                    output_weight=output_weight)
        if output_bias is not None:
            expect["output_bias"] = (Cout,)
            args["output_bias"] = output_bias
        for name, shp in expect.items():
            t = args[name]
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
            args[name] = _prep(t, f32, dev, name)
        if frame_mask is None:
            raise ValueError("frame_mask [B,N] is required")
        if tuple(frame_mask.shape) != (B, N) or frame_mask.device != dev:
            raise ValueError(f"frame_mask must be [B,N] = {(B, N)} on {dev}")
        fm = frame_mask.to(torch.uint8).contiguous()
        pm, strides = None, None
        if pair_mask is not None:
            if pair_mask.device != dev:
                raise ValueError(f"pair_mask is on {pair_mask.device}, expected {dev}")
            pm = pair_mask if pair_mask.dtype == torch.uint8 else pair_mask.to(torch.uint8)
            pm = pm.expand(B, H, N, N)               # broadcast dims get stride 0
            strides = (ctypes.c_int64 * 4)(*pm.stride())
            pm_ptr = pm.data_ptr()
        stream = _order_on(stream, dev, [*args.values(), fm, pm, self.workspace, self.vectors,
                                         self.output, self.attention])
        self.bound = (args, fm, pm, strides)
        return (ctypes.byref(self.dims),
                *(args[n].data_ptr() for n in ("rot", "trans", "q_direction", "k_direction",
                                               "q_point", "k_point", "values", "direction_scale",
                                               "distance_scale", "output_weight")),
                _dev_ptr(args.get("output_bias")), fm.data_ptr(),
                pm_ptr if pm is not None else 0,
                ctypes.cast(strides, ctypes.c_void_p) if strides is not None else None,
                self.vectors.data_ptr(), self.output.data_ptr(), _dev_ptr(self.attention),
                self.workspace.data_ptr(), ctypes.c_size_t(self.ws_bytes),
                ctypes.c_void_p(stream.cuda_stream))

    def forward_raw(self, raw: tuple) -> dict:
        rc = self.lib.ipa_dirdist_forward(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))
        out = {"vectors": self.vectors, "output": self.output}
        if self.attention is not None:
            out["attention"] = self.attention
        return out

    def __call__(self, *args, **kw) -> dict:
        return self.forward_raw(self.bind(*args, **kw))


def geometric_reasoning_attention(rot, trans, q_direction, k_direction, q_point, k_point, values,
                                  direction_scale, distance_scale, output_weight, output_bias=None,
                                  frame_mask=None, pair_mask=None, attention=True) -> dict:
    """Direction-and-distance attention on the device of ``values``.
    Returns freshly allocated float32 tensors: "vectors" [B,N,H,M,3],
    "output" [B,N,Cout] and, if ``attention``, "attention" [B,H,N,N]."""
    B, N, H, M, _ = values.shape
    Cout = output_weight.shape[1]
    plan = DirDistForward(B, N, H, M, Cout, device=values.device, attention=attention)
    return plan(rot, trans, q_direction, k_direction, q_point, k_point, values, direction_scale,
                distance_scale, output_weight, output_bias, frame_mask, pair_mask)


# ---------------------------------------------------------------------------
# gradient of the forward (ipa_backward, float32)
# ---------------------------------------------------------------------------
BACKWARD_INPUTS = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "z1", "z2", "w_b", "gamma")


def backward_workspace_bytes(B, L, H, C, Pqk, Pv, R, Cz) -> int:
    d = make_dims(B, L, H, C, Pqk, Pv, R, Cz)
    return int(load_library().ipa_backward_workspace_bytes(ctypes.byref(d)))


class IPABackward:
    """Reusable plan of the IPA gradient (ipa_backward, float32): validated
    shapes, preallocated workspace and gradient tensors on one device."""

    def __init__(self, B, L, H, C, Pqk, Pv, R, Cz, device=None):
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = make_dims(B, L, H, C, Pqk, Pv, R, Cz)
        self.shape = dict(B=B, L=L, H=H, C=C, Pqk=Pqk, Pv=Pv, R=R, Cz=Cz)
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_backward_workspace_bytes(ctypes.byref(self.dims)))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape}")
        dev, f32 = self.device, torch.float32
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.shapes = {"q": (B, L, H, C), "k": (B, L, H, C), "v": (B, L, H, C),
                       "q_pts": (B, L, H, Pqk, 3), "k_pts": (B, L, H, Pqk, 3), "v_pts": (B, L, H, Pv, 3),
                       "rot": (B, L, 3, 3), "trans": (B, L, 3), "z1": (B, L, R, Cz), "z2": (B, L, R, Cz),
                       "w_b": (Cz, H), "gamma": (H,)}
        self.grads = {n: torch.empty(shp, dtype=f32, device=dev) for n, shp in self.shapes.items()}

    # storage dtype of each input (the flash form may take bf16 features)
    def _in_dtype(self, name: str) -> torch.dtype:
        return torch.float32

    def bind(self, inputs: dict, outputs: dict, cotangents: dict, mask=None, w_L=None, w_C=None,
             stream=None) -> tuple:
        B, L, H, C, Pv, Cz = (self.shape[n] for n in ("B", "L", "H", "C", "Pv", "Cz"))
        dev, f32 = self.device, torch.float32
        if w_L is None or w_C is None:
            dl, dc = default_weights(self.shape["Pqk"])
            w_L = dl if w_L is None else w_L
            w_C = dc if w_C is None else w_C
        t = {}
        for n, shp in self.shapes.items():
            x = inputs[n]
            if tuple(x.shape) != shp:
                raise ValueError(f"{n} has shape {tuple(x.shape)}, expected {shp}")
            t[n] = _prep(x, self._in_dtype(n), dev, n)
        oshapes = {"s": (B, L, H, C), "pts": (B, L, H, Pv, 3), "pts_norm": (B, L, H, Pv), "pair": (B, L, H, Cz)}
        o = {n: _prep(outputs[n], f32, dev, "out_" + n) for n in ("s", "pts", "pair")}
        g = {}
        for n, shp in oshapes.items():
            x = cotangents[n]
            if tuple(x.shape) != shp:
                raise ValueError(f"cotangent {n} has shape {tuple(x.shape)}, expected {shp}")
            g[n] = _prep(x, f32, dev, "g_" + n)
        m = None
        if mask is not None:
            m = (mask.to(torch.uint8) if mask.dtype != torch.uint8 else mask).contiguous()
        stream = _order_on(stream, dev, [*t.values(), *o.values(), *g.values(), m, self.workspace,
                                         *self.grads.values()])
        self.bound = (t, o, g, m)
        return (ctypes.byref(self.dims), *(t[n].data_ptr() for n in BACKWARD_INPUTS), _dev_ptr(m),
                ctypes.c_float(w_L), ctypes.c_float(w_C),
                o["s"].data_ptr(), o["pts"].data_ptr(), o["pair"].data_ptr(),
                g["s"].data_ptr(), g["pts"].data_ptr(), g["pts_norm"].data_ptr(), g["pair"].data_ptr(),
                *(self.grads[n].data_ptr() for n in BACKWARD_INPUTS),
                self.workspace.data_ptr(), ctypes.c_size_t(self.ws_bytes), ctypes.c_void_p(stream.cuda_stream))

    def backward_raw(self, raw: tuple) -> dict:
        rc = self.lib.ipa_backward(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))
        return self.grads

    def __call__(self, *args, **kw) -> dict:
        return self.backward_raw(self.bind(*args, **kw))


def backward_flash_workspace_bytes(B, L, H, C, Pqk, Pv, R, Cz) -> int:
    d = make_dims(B, L, H, C, Pqk, Pv, R, Cz)
    return int(load_library().ipa_backward_flash_workspace_bytes(ctypes.byref(d)))


class IPABackwardFlash(IPABackward):
    """Reusable plan of the IPA gradient in flash form (ipa_backward_flash):
    no score rows are stored, the workspace is linear in L. ``dtype`` is the
    storage of q, k, v, the points, z1 and z2 (torch.bfloat16 or
    torch.float32); frames, W_b, gamma, outputs, cotangents and gradients are
    float32."""

    _FEATURES = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "z1", "z2")

    def __init__(self, B, L, H, C, Pqk, Pv, R, Cz, dtype=torch.bfloat16, device=None):
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be torch.bfloat16 or torch.float32")
        self.in_dtype = dtype
        self.code = IPA_BF16 if dtype == torch.bfloat16 else IPA_F32
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = make_dims(B, L, H, C, Pqk, Pv, R, Cz)
        self.shape = dict(B=B, L=L, H=H, C=C, Pqk=Pqk, Pv=Pv, R=R, Cz=Cz)
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_backward_flash_workspace_bytes(ctypes.byref(self.dims)))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape}")
        dev, f32 = self.device, torch.float32
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.shapes = {"q": (B, L, H, C), "k": (B, L, H, C), "v": (B, L, H, C),
                       "q_pts": (B, L, H, Pqk, 3), "k_pts": (B, L, H, Pqk, 3), "v_pts": (B, L, H, Pv, 3),
                       "rot": (B, L, 3, 3), "trans": (B, L, 3), "z1": (B, L, R, Cz), "z2": (B, L, R, Cz),
                       "w_b": (Cz, H), "gamma": (H,)}
        self.grads = {n: torch.empty(shp, dtype=f32, device=dev) for n, shp in self.shapes.items()}

    def _in_dtype(self, name: str) -> torch.dtype:
        return self.in_dtype if name in self._FEATURES else torch.float32

    def bind(self, *args, **kw) -> tuple:
        raw = super().bind(*args, **kw)
        return (raw[0], ctypes.c_int32(self.code), *raw[1:])

    def backward_raw(self, raw: tuple) -> dict:
        rc = self.lib.ipa_backward_flash(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))
        return self.grads


# ---------------------------------------------------------------------------
# the full layer (ipa_layer_forward)
# ---------------------------------------------------------------------------
class IPALayer:
    """Reusable plan of the full IPA layer (ipa_layer_forward): projections
    of the single representation, the attention, the readout."""

    def __init__(self, B, L, H, C, Pqk, Pv, R, Cz, c_s, dtype=torch.bfloat16, device=None):
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be torch.bfloat16 or torch.float32")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dims = make_dims(B, L, H, C, Pqk, Pv, R, Cz)
        self.shape = dict(B=B, L=L, H=H, C=C, Pqk=Pqk, Pv=Pv, R=R, Cz=Cz, c_s=c_s)
        self.code = IPA_BF16 if dtype == torch.bfloat16 else IPA_F32
        self.lib = load_library()
        self.ws_bytes = int(self.lib.ipa_layer_workspace_bytes(ctypes.byref(self.dims), c_s, self.code))
        if self.ws_bytes == 0:
            raise IPAError(-6, f"unsupported dims {self.shape} for {dtype}")
        self.n_in = 3 * H * C + 6 * H * Pqk + 3 * H * Pv + 2 * R * Cz
        self.n_out = H * (C + 4 * Pv + Cz)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.out = torch.empty(B, L, c_s, dtype=torch.float32, device=self.device)

    def bind(self, s, rot, trans, w_in, b_in, w_b, gamma, w_out, b_out, mask=None, w_L=None, w_C=None,
             stream=None) -> tuple:
        B, L, H, Cz, c_s = (self.shape[n] for n in ("B", "L", "H", "Cz", "c_s"))
        dev, f32 = self.device, torch.float32
        if w_L is None or w_C is None:
            dl, dc = default_weights(self.shape["Pqk"])
            w_L = dl if w_L is None else w_L
            w_C = dc if w_C is None else w_C
        expect = {"s": (B, L, c_s), "rot": (B, L, 3, 3), "trans": (B, L, 3), "w_in": (c_s, self.n_in),
                  "w_b": (Cz, H), "gamma": (H,), "w_out": (self.n_out, c_s)}
        args = dict(s=s, rot=rot, trans=trans, w_in=w_in, w_b=w_b, gamma=gamma, w_out=w_out)
        for name, shp in expect.items():
            t = args[name]
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
            args[name] = _prep(t, f32, dev, name)
        bi = _prep(b_in, f32, dev, "b_in") if b_in is not None else None
        bo = _prep(b_out, f32, dev, "b_out") if b_out is not None else None
        m = None
        if mask is not None:
            m = (mask.to(torch.uint8) if mask.dtype != torch.uint8 else mask).contiguous()
        stream = _order_on(stream, dev, [*args.values(), bi, bo, m, self.workspace, self.out])
        self.bound = (args, bi, bo, m)
        return (ctypes.byref(self.dims), self.shape["c_s"], self.code,
                args["s"].data_ptr(), args["rot"].data_ptr(), args["trans"].data_ptr(), _dev_ptr(m),
                args["w_in"].data_ptr(), _dev_ptr(bi), args["w_b"].data_ptr(), args["gamma"].data_ptr(),
                ctypes.c_float(w_L), ctypes.c_float(w_C), args["w_out"].data_ptr(), _dev_ptr(bo),
                self.out.data_ptr(), self.workspace.data_ptr(), ctypes.c_size_t(self.ws_bytes),
                ctypes.c_void_p(stream.cuda_stream))

    def forward_raw(self, raw: tuple) -> torch.Tensor:
        rc = self.lib.ipa_layer_forward(*raw)
        if rc != 0:
            raise IPAError(rc, status_string(rc))
        return self.out

    def __call__(self, *args, **kw) -> torch.Tensor:
        return self.forward_raw(self.bind(*args, **kw))
