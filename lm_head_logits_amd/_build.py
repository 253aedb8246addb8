"""Compile the HIP library in-tree: lm_head_logits_amd/liblmhead.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "liblmhead.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    # no packed-fp32 VALU code: those forms are not used on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def build(verbose: bool = False) -> Path:
    """Always recompiles (a stale library must never be picked up)."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", str(PKG.parent / "include"), "-o", str(tmp),
           *map(str, sources())]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
