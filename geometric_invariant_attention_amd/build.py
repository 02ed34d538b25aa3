"""Build the HIP library libipa_mi355.so (gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB_NAME = "libipa_mi355.so"
LIB_PATH = PKG / LIB_NAME
BUILD_DIR = PKG / "_build"

SOURCES = ["ipa_api.cpp", "ipa_lift.hip", "ipa_attn.hip", "ipa_frames.hip", "ipa_dirdist.hip", "ipa_bwd.hip", "ipa_bwd_flash.hip", "ipa_gemm.hip", "ipa_layer.hip", "ipa_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"),
]

# Per-source extra flags (none at present).
EXTRA_FLAGS: dict[str, list[str]] = {}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the IPA library)")


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    """Compile every source for gfx950 and link the shared library."""
    hipcc = _hipcc()
    BUILD_DIR.mkdir(exist_ok=True)
    objs = []

    def compile_one(src: str) -> Path:
        obj = BUILD_DIR / (src + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", str(CSRC / src), "-o", str(obj)]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=jobs or min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
