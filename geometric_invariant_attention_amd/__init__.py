"""Fused invariant point attention (IPA) forward for AMD MI355X (gfx950).

The computation lives in the HIP library ``libipa_mi355.so`` (C ABI in
``include/ipa.h``); this package only marshals torch tensors into it.
"""

from ._binding import (  # noqa: F401
    IPA_BF16, IPA_F32, IPAError, IPAForward, IpaDims, LIB_PATH, default_weights,
    ipa_forward, load_library, make_dims, status_string, workspace_bytes,
    frames_from_atoms, meet_attention, MeetForward, IpaMeetDims, meet_workspace_bytes,
    DirDistForward, IpaDirDistDims, dirdist_workspace_bytes, geometric_reasoning_attention,
    IPABackward, backward_workspace_bytes, IPALayer,
    IPABackwardFlash, backward_flash_workspace_bytes,
)

__all__ = ["ipa_forward", "IPAForward", "IPAError", "load_library", "workspace_bytes",
           "status_string", "make_dims", "IpaDims", "default_weights", "IPA_F32",
           "IPA_BF16", "LIB_PATH", "frames_from_atoms", "meet_attention", "MeetForward",
           "IpaMeetDims", "meet_workspace_bytes", "DirDistForward", "IpaDirDistDims",
           "dirdist_workspace_bytes", "geometric_reasoning_attention", "IPABackward",
           "backward_workspace_bytes", "IPALayer", "IPABackwardFlash",
           "backward_flash_workspace_bytes"]
