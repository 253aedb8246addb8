"""The tiled kernel's generated code hands each LDS stage over only after the
direct-to-LDS loads that fill it have landed (CPU: compiles to assembly).

The waves of a work-group load one shared stage with direct-to-LDS loads and
then read each other's rows; the barrier between must be preceded by a vmcnt
wait that retires those loads, or a wave may read rows still in flight. The
kernel waits explicitly for the 16-bit weight path and relies on the
compiler's barrier (vmcnt of the later code loads) for the NVFP4 path; both
are checked here on every instantiation.
"""
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT / "tests"))
from asm_check import barriers_with_pending_lds_loads, kernel_bodies  # noqa: E402


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    return None


@pytest.fixture(scope="module")
def tiled_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    import importlib.util
    spec = importlib.util.spec_from_file_location("lmhead_build", ROOT / "lm_head_logits_amd" / "_build.py")
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared",)]
    out = tmp_path_factory.mktemp("asm") / "tiled.s"
    cmd = [hipcc, *flags, "-S", "--cuda-device-only", "-I", str(ROOT / "include"), "-o", str(out),
           str(ROOT / "lm_head_logits_amd" / "csrc" / "tiled.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_every_stage_barrier_retires_the_direct_loads(tiled_asm):
    kernels = {k: v for k, v in kernel_bodies(tiled_asm).items() if "tiled_kernel" in k}
    assert len(kernels) >= 20  # 16-bit and NVFP4 instantiations
    seen_lds_loads = 0
    for name, (lines, labels) in kernels.items():
        n_lds = sum(1 for t in lines if t.startswith("buffer_load") and t.endswith(" lds"))
        n_bar = sum(1 for t in lines if t == "s_barrier")
        assert n_lds > 0 and n_bar > 0, name
        seen_lds_loads += n_lds
        bad = barriers_with_pending_lds_loads(lines, labels)
        assert not bad, f"{name}: barrier(s) at {bad} may run before direct-to-LDS loads land"
    assert seen_lds_loads > 0


# The checker itself, on hand-written sequences.

def _check(src):
    lines = [l.strip() for l in src.strip().splitlines()]
    body = [l for l in lines if not l.endswith(":")]
    labels = {}
    k = 0
    for l in lines:
        if l.endswith(":"):
            labels[l[:-1]] = k
        else:
            k += 1
    return barriers_with_pending_lds_loads(body, labels)


def test_checker_flags_a_barrier_without_vmcnt():
    assert _check("""
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
        s_waitcnt lgkmcnt(0)
        s_barrier
        s_endpgm""") == [2]


def test_checker_accepts_vmcnt_that_retires_the_load():
    # one later load: vmcnt(1) retires the direct load, vmcnt(2) does not
    ok = """
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
        buffer_load_dwordx4 v[2:5], v1, s[0:3], 0 offen
        s_waitcnt vmcnt(1) lgkmcnt(0)
        s_barrier
        s_endpgm"""
    assert _check(ok) == []
    assert _check(ok.replace("vmcnt(1)", "vmcnt(2)")) == [3]


def test_checker_follows_loop_back_edges():
    # the load at the end of the loop body reaches the barrier at its top
    assert _check("""
        s_waitcnt vmcnt(0)
        .LBB0_1:
        s_barrier
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
        s_cbranch_scc1 .LBB0_1
        s_endpgm""") == [1]
