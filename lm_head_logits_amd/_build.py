"""Compile the HIP libraries in-tree (gfx950): lm_head_logits_amd/liblmhead.so,
the projection, and lm_head_logits_amd/liblmhead_probes.so, the measurement
probes the benchmark reports alongside it (not part of the projection)."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "liblmhead.so"
PROBES_SRC = PKG / "probes"
PROBES_LIB = PKG / "liblmhead_probes.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
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


def probe_sources():
    return sorted(PROBES_SRC.glob("*.hip"))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    noise = "is not a recognized feature for this target"
    return r.returncode, [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]


def build(verbose: bool = False) -> Path:
    """Always recompiles (a stale library must never be picked up). Each source
    is compiled to its own object in parallel, then each library's objects
    are linked. Returns the projection's library."""
    inc = ["-I", str(PKG.parent / "include")]
    srcs = sources() + probe_sources()
    libs = ((LIB, [s.name for s in sources()]), (PROBES_LIB, [s.name for s in probe_sources()]))
    with tempfile.TemporaryDirectory(prefix="lmhead_build_") as d:
        objs = [str(Path(d) / (s.name + ".o")) for s in srcs]
        cmds = [[hipcc(), *HIPCC_FLAGS, *inc, "-c", str(s), "-o", o] for s, o in zip(srcs, objs)]
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        msgs = []
        for cmd, (rc, m) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            msgs += m
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {cmd[-3]}:\n" + "\n".join(m))
        for lib, names in libs:
            tmp = lib.with_suffix(".so.tmp")
            mine = [str(Path(d) / (n + ".o")) for n in names]
            rc, m = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *mine])
            msgs += m
            if rc != 0:
                raise RuntimeError(f"link of {lib.name} failed:\n" + "\n".join(m))
            os.replace(tmp, lib)
    if verbose and msgs:
        print("\n".join(msgs))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
