"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspace linearly in L, and rejects bad
arguments before anything is launched."""

import ctypes
import re
from pathlib import Path

import pytest

from geometric_invariant_attention_amd import _binding as bd

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ipa.h"


@pytest.fixture(scope="module")
def lib():
    if not bd.LIB_PATH.exists():
        pytest.skip("HIP library not built (run __graft_entry__.build())")
    return bd.load_library()


def _declared():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ipa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert names == ["ipa_attend", "ipa_backward", "ipa_backward_flash",
                     "ipa_backward_flash_workspace_bytes", "ipa_backward_workspace_bytes",
                     "ipa_dirdist_forward", "ipa_dirdist_workspace_bytes",
                     "ipa_forward", "ipa_forward_noalloc", "ipa_frames_from_atoms", "ipa_layer_forward",
                     "ipa_layer_workspace_bytes", "ipa_lift",
                     "ipa_meet_forward", "ipa_meet_workspace_bytes", "ipa_status_string",
                     "ipa_version", "ipa_workspace_bytes"]
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.ipa_version() >= 100
    for code in list(bd.STATUS) + [-99]:
        s = bd.status_string(code)
        assert isinstance(s, str) and s


def _dims(**kw):
    base = dict(B=1, L=512, H=12, C=16, Pqk=4, Pv=8, R=2, Cz=128)
    base.update(kw)
    return bd.IpaDims(**base)


def test_workspace_linear_in_L(lib):
    sizes = {L: bd.workspace_bytes(_dims(L=L), bd.IPA_BF16) for L in (1024, 2048, 4096, 8192, 16384)}
    assert all(v > 0 for v in sizes.values())
    # exactly linear for multiples of the tile sizes (no L*L term)
    per = (sizes[16384] - sizes[8192]) / 8192
    for L, v in sizes.items():
        assert abs(v - sizes[1024] - per * (L - 1024)) < 4096, (L, v)
    # modest: about 6 KB per residue at H=12, c_z=128 in bf16
    assert per < 8192


@pytest.mark.parametrize("kw,dtype", [
    (dict(L=0), bd.IPA_BF16), (dict(H=-1), bd.IPA_BF16), (dict(C=17), bd.IPA_BF16),
    (dict(Pqk=6), bd.IPA_BF16), (dict(Pv=9), bd.IPA_BF16), (dict(Cz=12), bd.IPA_BF16),
    (dict(Cz=256, R=1), bd.IPA_BF16), (dict(R=3), bd.IPA_BF16), (dict(R=2), bd.IPA_F32),
    (dict(), 7),
])
def test_workspace_zero_when_unsupported(lib, kw, dtype):
    assert bd.workspace_bytes(_dims(**kw), dtype) == 0


def _call(lib, dims, dtype=bd.IPA_BF16, ptr=0x100000, ws_bytes=1 << 40, w_L=0.5, w_C=0.3,
          null_idx=None, misalign_idx=None, ws_ptr=None):
    """Call ipa_forward with fake device pointers. Every case used here fails
    validation, so nothing is ever launched."""
    ptrs = [ptr + 4096 * i for i in range(13)]
    outs = [ptr + 4096 * (13 + i) for i in range(4)]
    allp = ptrs + outs
    if null_idx is not None:
        allp[null_idx] = 0
    if misalign_idx is not None:
        allp[misalign_idx] += 4
    ws = ptr + (1 << 30) if ws_ptr is None else ws_ptr
    d = ctypes.byref(dims) if dims is not None else None
    return lib.ipa_forward(d, dtype, *allp[:12], 0, ctypes.c_float(w_L), ctypes.c_float(w_C),
                           *allp[13:17], ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("entry", ["ipa_forward", "ipa_lift", "ipa_attend"])
def test_stages_reject_before_launch(lib, entry):
    fn = getattr(lib, entry)
    d = _dims()
    assert fn(None, 1, *([0x100000] * 12), 0, ctypes.c_float(0.5), ctypes.c_float(0.3),
              *([0x200000] * 4), 0x40000000, ctypes.c_size_t(1 << 40), None) == -1
    assert fn(ctypes.byref(d), 1, *([0x100000] * 12), 0, ctypes.c_float(0.5), ctypes.c_float(0.3),
              *([0x200000] * 4), 0x40000000, ctypes.c_size_t(16), None) == -4


def test_forward_rejects_before_launch(lib):
    assert _call(lib, None) == -1                                  # IPA_ERR_NULL
    assert _call(lib, _dims(L=0)) == -2                            # IPA_ERR_DIMS
    assert _call(lib, _dims(), dtype=5) == -3                      # IPA_ERR_DTYPE
    for idx in (0, 5, 9, 11, 13, 16):
        assert _call(lib, _dims(), null_idx=idx) == -1             # NULL tensor
        assert _call(lib, _dims(), misalign_idx=idx) == -5         # IPA_ERR_ALIGN
    assert _call(lib, _dims(), ws_ptr=0x100000 + (1 << 30) + 16) == -5
    assert _call(lib, _dims(), w_L=float("nan")) == -8             # IPA_ERR_ARG
    assert _call(lib, _dims(), w_C=-1.0) == -8
    assert _call(lib, _dims(C=20)) == -6                           # IPA_ERR_UNSUPPORTED
    assert _call(lib, _dims(R=2, Cz=128), dtype=bd.IPA_F32) == -6
    need = bd.workspace_bytes(_dims(), bd.IPA_BF16)
    assert _call(lib, _dims(), ws_bytes=need - 1) == -4            # IPA_ERR_WORKSPACE


def test_noalloc_rejects_before_launch(lib):
    """ipa_forward_noalloc refuses dims beyond its static workspace, and
    reports invalid arguments as ipa_forward does, before any HIP call."""
    def call(dims, dtype=bd.IPA_BF16):
        d = ctypes.byref(dims) if dims is not None else None
        return lib.ipa_forward_noalloc(d, dtype, *([0x100000] * 12), None, ctypes.c_float(0.5),
                                       ctypes.c_float(0.3), *([0x200000] * 4), None)
    limit = 64 << 20
    big = _dims(L=16384, H=8)
    assert bd.workspace_bytes(big, bd.IPA_BF16) > limit
    assert call(big) == -9                                          # IPA_ERR_LIMIT
    assert "IPA_NOALLOC_WORKSPACE_BYTES" in bd.status_string(-9)
    assert bd.workspace_bytes(_dims(L=8192), bd.IPA_BF16) <= limit
    assert call(None) == -1
    assert call(_dims(L=0)) == -2
    assert call(_dims(), dtype=5) == -3
    assert call(_dims(C=20)) == -6


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        bd.load_library(tmp_path / "missing.so")


def test_frames_reject_before_launch(lib):
    f = lib.ipa_frames_from_atoms
    good = [0x100000 + 4096 * i for i in range(5)]
    assert f(0, 4, *good, None) == -2                              # IPA_ERR_DIMS
    assert f(1, 0, *good, None) == -2
    assert f(1 << 16, 1 << 15, *good, None) == -2                  # B*L >= 2^31
    for idx in range(5):
        bad = list(good)
        bad[idx] = 0
        assert f(1, 4, *bad, None) == -1                           # IPA_ERR_NULL
        bad = list(good)
        bad[idx] += 2
        assert f(1, 4, *bad, None) == -5                           # IPA_ERR_ALIGN


def _meet_call(lib, dims, dtype=bd.IPA_BF16, null_idx=None, misalign_idx=None, ws_bytes=1 << 40, ws_ptr=None):
    """ipa_meet_forward with fake device pointers; every case fails validation."""
    ptrs = [0x100000 + 4096 * i for i in range(7)]     # q, k, v, x, rho, s, out
    if null_idx is not None:
        ptrs[null_idx] = 0
    if misalign_idx is not None:
        ptrs[misalign_idx] += 4
    ws = 0x40000000 if ws_ptr is None else ws_ptr
    d = ctypes.byref(dims) if dims is not None else None
    return lib.ipa_meet_forward(d, dtype, *ptrs[:6], 0, ptrs[6], ws, ctypes.c_size_t(ws_bytes), None)


def test_meet_rejects_before_launch(lib):
    d = bd.IpaMeetDims(1, 512, 12, 16)
    assert _meet_call(lib, None) == -1
    assert _meet_call(lib, bd.IpaMeetDims(1, 0, 12, 16)) == -2
    assert _meet_call(lib, d, dtype=5) == -3
    for idx in range(7):
        assert _meet_call(lib, d, null_idx=idx) == -1
        assert _meet_call(lib, d, misalign_idx=idx) == -5
    assert _meet_call(lib, d, ws_ptr=0x40000000 + 16) == -5
    assert _meet_call(lib, bd.IpaMeetDims(1, 512, 12, 17)) == -6
    need = bd.meet_workspace_bytes(1, 512, 12, 16, bd.IPA_BF16)
    assert need > 0
    assert _meet_call(lib, d, ws_bytes=need - 1) == -4


def test_meet_workspace_linear_in_L(lib):
    sizes = {L: bd.meet_workspace_bytes(1, L, 8, 16, bd.IPA_BF16) for L in (1024, 2048, 4096, 8192)}
    per = (sizes[8192] - sizes[4096]) / 4096
    for L, v in sizes.items():
        assert abs(v - sizes[1024] - per * (L - 1024)) < 4096, (L, v)
    assert bd.meet_workspace_bytes(1, 64, 4, 0, bd.IPA_F32) == 0


def _dd_call(lib, dims, ptrs=None, ws_bytes=1 << 30, ws=0x100000, strides=None, pm=0):
    """ipa_dirdist_forward with fake device pointers; every case fails
    validation before a launch."""
    d = bd.IpaDirDistDims(*dims) if dims is not None else None
    if ptrs is None:
        ptrs = [0x1000 * (n + 1) for n in range(15)]
    st = (ctypes.c_int64 * 4)(*strides) if strides is not None else None
    return lib.ipa_dirdist_forward(ctypes.byref(d) if d is not None else None,
                                   *ptrs[:11], ptrs[11], pm,
                                   ctypes.cast(st, ctypes.c_void_p) if st is not None else None,
                                   ptrs[12], ptrs[13], ptrs[14], ws, ctypes.c_size_t(ws_bytes), None)


def test_dirdist_rejects_before_launch(lib):
    good = (1, 64, 4, 4, 16)
    assert _dd_call(lib, None) == -1
    assert _dd_call(lib, (0, 64, 4, 4, 16)) == -2
    assert _dd_call(lib, (1, 64, 4, 9, 16)) == -6            # M > 8
    assert _dd_call(lib, (1, 64, 4, 4, 70000)) == -6         # Cout > 65536
    for k in range(10):                                      # each required float input
        p = [0x1000 * (n + 1) for n in range(15)]
        p[k] = 0
        assert _dd_call(lib, good, p) == -1, k
    p = [0x1000 * (n + 1) for n in range(15)]
    p[11] = 0                                                # frame mask
    assert _dd_call(lib, good, p) == -1
    p = [0x1000 * (n + 1) for n in range(15)]
    p[12] = 0                                                # vectors
    assert _dd_call(lib, good, p) == -1
    p = [0x1000 * (n + 1) for n in range(15)]
    p[3] += 2                                                # misaligned float
    assert _dd_call(lib, good, p) == -5
    assert _dd_call(lib, good, ws=0x100010) == -5            # workspace alignment
    need = lib.ipa_dirdist_workspace_bytes(ctypes.byref(bd.IpaDirDistDims(*good)))
    assert _dd_call(lib, good, ws_bytes=need - 1) == -4
    assert _dd_call(lib, good, pm=0x9000) == -1              # mask without strides
    assert _dd_call(lib, good, pm=0x9000, strides=(0, 0, 64, -1)) == -8


def test_dirdist_workspace_linear_in_N(lib):
    def ws(N):
        return lib.ipa_dirdist_workspace_bytes(ctypes.byref(bd.IpaDirDistDims(1, N, 8, 4, 64)))
    # linear once the chip is full without splitting the keys (N >= 8192 here)
    a, b, c = ws(8192), ws(16384), ws(32768)
    assert a > 0 and abs((c - b) - 2 * (b - a)) <= 4 * 256
    # and bounded by a multiple of N below that (the key splits add partials)
    per = [ws(n) / n for n in (64, 256, 1024, 2048, 4096, 8192)]
    assert max(per) <= 3 * per[-1]
    assert lib.ipa_dirdist_workspace_bytes(ctypes.byref(bd.IpaDirDistDims(1, 64, 4, 9, 16))) == 0


def test_backward_rejects_before_launch(lib):
    good = bd.make_dims(1, 64, 4, 16, 4, 8, 2, 16)
    ptrs = [0x1000 * (n + 1) for n in range(33)]

    def call(dims, p=ptrs, mask=0, wl=1.0, wc=1.0, ws_bytes=1 << 34, ws=0x100000):
        return lib.ipa_backward(ctypes.byref(dims) if dims is not None else None, *p[:12], mask,
                                ctypes.c_float(wl), ctypes.c_float(wc), *p[12:31], ws,
                                ctypes.c_size_t(ws_bytes), None)
    assert call(None) == -1
    assert call(bd.make_dims(1, 0, 4, 16, 4, 8, 2, 16)) == -2
    assert call(bd.make_dims(1, 64, 4, 32, 4, 8, 2, 16)) == -6       # C > 16
    assert call(bd.make_dims(1, 64, 4, 16, 4, 8, 4, 128)) == -6      # R Cz > 256
    for k in range(31):
        p = list(ptrs)
        p[k] = 0
        assert call(good, p) == -1, k
    p = list(ptrs)
    p[5] += 2
    assert call(good, p) == -5
    assert call(good, ws=0x100010) == -5
    assert call(good, wl=float("nan")) == -8
    need = lib.ipa_backward_workspace_bytes(ctypes.byref(good))
    assert need > 0 and call(good, ws_bytes=need - 1) == -4


def test_backward_workspace_linear_in_L(lib):
    """The per-row arrays grow linearly in L; the two score buffers of a
    query chunk are capped at 2^26 floats each, so past the cap the whole
    workspace grows at most linearly."""
    def ws(L):
        return lib.ipa_backward_workspace_bytes(ctypes.byref(bd.make_dims(1, L, 12, 16, 4, 8, 2, 128)))
    sizes = {L: ws(L) for L in (1024, 4096, 8192, 16384, 32768, 65536)}
    assert all(v > 0 for v in sizes.values())
    for L in (4096, 8192, 16384, 32768):
        assert sizes[2 * L] <= 2 * sizes[L]
    # the score buffers never exceed 2 x 2^26 floats: past the cap, doubling
    # L adds less than the per-row arrays of L more rows plus the buffers
    grow = sizes[65536] - sizes[32768]
    assert sizes[65536] <= 2 * grow + 2 * 4 * (1 << 26) + 17 * 256


def test_backward_flash_rejects_before_launch(lib):
    good = bd.make_dims(1, 64, 4, 16, 4, 8, 2, 16)
    ptrs = [0x1000 * (n + 1) for n in range(33)]

    def call(dims, dtype=1, p=ptrs, mask=0, wl=1.0, wc=1.0, ws_bytes=1 << 34, ws=0x100000):
        return lib.ipa_backward_flash(ctypes.byref(dims) if dims is not None else None, dtype, *p[:12], mask,
                                      ctypes.c_float(wl), ctypes.c_float(wc), *p[12:31], ws,
                                      ctypes.c_size_t(ws_bytes), None)
    assert call(None) == -1
    assert call(bd.make_dims(1, 0, 4, 16, 4, 8, 2, 16)) == -2
    assert call(good, dtype=2) == -3
    assert call(bd.make_dims(1, 64, 4, 32, 4, 8, 2, 16)) == -6       # C > 16
    assert call(bd.make_dims(1, 64, 4, 16, 6, 8, 2, 16)) == -6       # Pqk > 5
    assert call(bd.make_dims(1, 64, 4, 16, 4, 8, 4, 128)) == -6      # R Cz > 256
    for k in range(31):
        p = list(ptrs)
        p[k] = 0
        assert call(good, p=p) == -1, k
    p = list(ptrs)
    p[5] += 2                       # bf16 features need 2-byte alignment only
    assert call(good, p=p, ws_bytes=0) == -4
    assert call(good, dtype=0, p=p) == -5
    p = list(ptrs)
    p[6] += 2                       # rot is float32 in either storage
    assert call(good, p=p) == -5
    assert call(good, ws=0x100010) == -5
    assert call(good, wl=float("nan")) == -8
    need = lib.ipa_backward_flash_workspace_bytes(ctypes.byref(good))
    assert need > 0 and call(good, ws_bytes=need - 1) == -4


def test_backward_flash_workspace_linear_in_L(lib):
    """The flash form stores no score rows: every buffer is a per-row
    array, so the workspace is a * L + b up to the 256-byte alignment of its
    17 buffers."""
    def ws(L):
        return lib.ipa_backward_flash_workspace_bytes(ctypes.byref(bd.make_dims(1, L, 12, 16, 4, 8, 2, 128)))
    Ls = (1024, 2048, 4096, 8192, 16384, 32768, 65536)
    sizes = [ws(L) for L in Ls]
    assert all(v > 0 for v in sizes)
    per_row = (sizes[-1] - sizes[0]) / (Ls[-1] - Ls[0])
    for L, v in zip(Ls, sizes):
        assert abs(v - (sizes[0] + per_row * (L - Ls[0]))) <= 17 * 256, (L, v)
    # about 93 KB per residue at 12 heads (bf16 lifted rows, fp32 lifted
    # gradients and the pair sums U): 6 GB at L = 65536
    assert per_row < 128 * 1024


def test_layer_rejects_before_launch(lib):
    good = bd.make_dims(1, 64, 4, 16, 4, 8, 2, 16)
    ptrs = [0x1000 * (n + 1) for n in range(16)]

    def call(dims, c_s=32, dtype=1, p=ptrs, wl=1.0, ws_bytes=1 << 34, ws=0x100000):
        return lib.ipa_layer_forward(ctypes.byref(dims) if dims is not None else None, c_s, dtype,
                                     *p[:8], ctypes.c_float(wl), ctypes.c_float(1.0), *p[8:11], ws,
                                     ctypes.c_size_t(ws_bytes), None)
    assert call(None) == -1
    assert call(good, c_s=0) == -2
    assert call(good, dtype=7) == -3
    for k in (0, 1, 2, 4, 6, 7, 8, 10):      # s, rot, trans, w_in, w_b, gamma, w_out, out
        p = list(ptrs)
        p[k] = 0
        assert call(good, p=p) == -1, k
    p = list(ptrs)
    p[4] += 4
    assert call(good, p=p) == -5
    assert call(good, wl=float("inf")) == -8
    need = lib.ipa_layer_workspace_bytes(ctypes.byref(good), 32, 1)
    assert need > 0 and call(good, ws_bytes=need - 1) == -4
    assert lib.ipa_layer_workspace_bytes(ctypes.byref(bd.make_dims(1, 64, 4, 32, 4, 8, 2, 16)), 32, 1) == 0
