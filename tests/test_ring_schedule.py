"""The weight-streaming kernels' explicit waits (CPU: host build and assembly).

The ring kernels (bf16 `skinny_kernel`, `nvfp4_ring_kernel`) wait for their
direct-to-LDS loads with compile-time vmcnt counts from `Schedule` and
`NvSchedule` (csrc/ring.hpp). Two checks:

- the counts equal those of a simulation of each kernel's issue order,
  written here from the kernels' code: at the first read of a unit, the
  number of loads issued after the last one the read needs (its two direct
  loads, and at a scale group's first chunk that group's scale loads); at the
  end of a chunk, the loads issued after the next chunk's hidden loads. A
  count one too large would let a read see a slot still in flight; one too
  small would only wait longer. Every (NB, NSL, HL) the launchers
  instantiate is checked over several periods, prologue included;
- in the generated code no direct-to-LDS load is issued while an LDS
  instruction of the same wave is outstanding (a direct load writes LDS on
  its own path, not behind the wave's earlier reads of the slot it refills).
"""
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "lm_head_logits_amd" / "csrc"
sys.path.insert(0, str(ROOT / "tests"))
from asm_check import kernel_bodies, lds_loads_with_pending_lds_ops  # noqa: E402

# (NB, NSL, HL) of every instantiation: the bf16 kernel with 4 or 8 waves of
# one block and 8 slots (HL = ceil(16 R * 8 / threads): 2 for R = 3, 4 with
# 256 threads), or 16 waves of up to 4 blocks and 4 slots (HL = 1); the NVFP4
# ring kernel with 16 waves of up to 3 blocks and 4 slots (HL = 1 for R <= 2).
BF16 = [(1, 8, 1), (1, 8, 2), (1, 4, 1), (2, 4, 1), (3, 4, 1), (4, 4, 1)]
NVFP4 = [(1, 4, 1), (2, 4, 1), (3, 4, 1)]

_PROG = r"""
#include "ring.hpp"
#include <cstdio>
using namespace lmhead;
template <int NB, int NSL, int HL> void bf() {
  using S = Schedule<NB, NSL, HL, 2>;
  std::printf("bf16 %d %d %d %d", NB, NSL, HL, S::PERIOD);
  for (int p = -1; p < S::PERIOD; ++p) std::printf(" %d,%d", p >= 0 ? S::wait_unit(p) : -1, S::wait_hidden(p));
  std::printf("\n");
}
template <int NB, int NSL, int HL> void nv() {
  using S = NvSchedule<NB, NSL, HL>;
  std::printf("nvfp4 %d %d %d %d", NB, NSL, HL, S::PERIOD);
  for (int p = -1; p < S::PERIOD; ++p) std::printf(" %d,%d", p >= 0 ? S::wait_first(p) : -1, S::wait_hidden(p));
  std::printf("\n");
}
int main() {
  %CALLS%
  return 0;
}
"""


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    return None


def _flags():
    import importlib.util
    spec = importlib.util.spec_from_file_location("lmhead_build", ROOT / "lm_head_logits_amd" / "_build.py")
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return [f for f in b.HIPCC_FLAGS if f not in ("-shared",)]


@pytest.fixture(scope="module")
def schedules(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("sched")
    calls = " ".join([f"bf<{a},{b},{c}>();" for a, b, c in BF16] +
                     [f"nv<{a},{b},{c}>();" for a, b, c in NVFP4])
    src = d / "dump.hip"
    src.write_text(_PROG.replace("%CALLS%", calls))
    exe = d / "dump"
    r = subprocess.run([hipcc, "--cuda-host-only", "-std=c++17", "-I", str(CSRC), "-I", str(ROOT / "include"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    res = {}
    for line in out.splitlines():
        kind, nb, nsl, hl, period, *vals = line.split()
        pairs = [tuple(int(x) for x in v.split(",")) for v in vals]
        res[(kind, int(nb), int(nsl), int(hl))] = (int(period), {p - 1: pairs[p] for p in range(len(pairs))})
    return res


class Issue:
    """The loads a wave has issued, in order, tagged."""

    def __init__(self):
        self.log = []

    def add(self, tag, n):
        self.log.extend([tag] * n)

    def after(self, tag):
        """Loads issued after the last one tagged `tag`."""
        last = max(i for i, t in enumerate(self.log) if t == tag)
        return len(self.log) - 1 - last


def simulate_bf16(NB, NSL, HL, units):
    """skinny_kernel: the prologue issues units 0 .. NSL-1 (two direct loads
    each) and, after a chunk's first unit, that chunk's HL hidden loads; then
    at each unit u: wait, read, issue unit u + NSL (and the hidden loads of
    the chunk it starts), and at a chunk's last unit wait for the next
    chunk's hidden loads."""
    q = Issue()
    for w in range(NSL):
        q.add(("u", w), 2)
        if w % NB == 0:
            q.add(("h", w // NB), HL)
    waits = {-1: (None, q.after(("h", 0)))}
    out = []
    for u in range(units):
        wu = q.after(("u", u))
        q.add(("u", u + NSL), 2)
        if (u + NSL) % NB == 0:
            q.add(("h", (u + NSL) // NB), HL)
        wh = q.after(("h", u // NB + 1)) if u % NB == NB - 1 else None
        out.append((u, wu, wh))
    return waits, out


def simulate_nvfp4(NB, NSL, HL, units):
    """nvfp4_ring_kernel: as the bf16 kernel, and each block's scales for a
    group of 8 chunks: issued after the unit that reads the group's last
    chunk (for the next group), the first group's in the prologue where the
    batches of units -NSL .. -1 sit in chunk -1. The first read of a group
    needs its scales as well as the unit's direct loads."""
    md = lambda a, m: ((a % m) + m) % m  # noqa: E731
    chunk = lambda v: v // NB  # floor, also for v < 0  # noqa: E731
    q = Issue()
    for w in range(NSL):
        vb = w - NSL
        q.add(("u", w), 2)
        if w % NB == 0:
            q.add(("h", w // NB), HL)
        if md(chunk(vb), 8) == 7:
            q.add(("s", md(vb, NB), 0), 2)
    waits = {-1: (None, q.after(("h", 0)))}
    out = []
    for u in range(units):
        j, c = u % NB, u // NB
        need = q.after(("u", u))
        if c % 8 == 0:
            need = min(need, q.after(("s", j, c // 8)))
        q.add(("u", u + NSL), 2)
        if (u + NSL) % NB == 0:
            q.add(("h", (u + NSL) // NB), HL)
        if c % 8 == 7:
            q.add(("s", j, c // 8 + 1), 2)
        wh = q.after(("h", c + 1)) if j == NB - 1 else None
        out.append((u, need, wh))
    return waits, out


@pytest.mark.parametrize("kind,params", [("bf16", p) for p in BF16] + [("nvfp4", p) for p in NVFP4])
def test_wait_counts_match_simulated_issue_order(schedules, kind, params):
    period, table = schedules[(kind,) + params]
    sim = simulate_bf16 if kind == "bf16" else simulate_nvfp4
    pro, steps = sim(*params, units=3 * period)
    assert table[-1][1] == pro[-1][1], "prologue wait for the first hidden chunk"
    for u, wu, wh in steps:
        p = u % period
        assert table[p][0] == wu, (kind, params, "unit", u)
        if wh is not None:
            assert table[p][1] == wh, (kind, params, "hidden", u)


def test_simulation_flags_a_wrong_count():
    # the comparison above would notice a schedule off by one load
    pro, steps = simulate_bf16(2, 4, 1, 8)
    assert any(wu > 0 for _, wu, _ in steps)
    pro2, steps2 = simulate_bf16(2, 4, 2, 8)  # one more hidden load per chunk
    assert [s[1] for s in steps] != [s[1] for s in steps2]


@pytest.fixture(scope="module")
def ring_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("ringasm")
    flags = _flags()

    def build(name):
        out = d / f"{name}.s"
        cmd = [hipcc, *flags, "-S", "--cuda-device-only", "-I", str(ROOT / "include"), "-o", str(out),
               str(CSRC / f"{name}.hip")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return out.read_text()

    with ThreadPoolExecutor(2) as ex:
        sk, nv = ex.map(build, ("skinny", "nvfp4"))
    return sk + nv


def test_no_direct_load_while_lds_ops_are_outstanding(ring_asm):
    kernels = {k: v for k, v in kernel_bodies(ring_asm).items()
               if "skinny_kernel" in k or "nvfp4_ring_kernel" in k}
    assert len(kernels) >= 60
    for name, (lines, labels) in kernels.items():
        n_dma = sum(1 for t in lines if t.startswith("buffer_load") and t.endswith(" lds"))
        assert n_dma > 0, name
        bad = lds_loads_with_pending_lds_ops(lines, labels)
        assert not bad, f"{name}: direct load(s) at {bad[:4]} issued with LDS reads in flight"


def _check(src):
    lines = [l.strip() for l in src.strip().splitlines()]
    body = [l for l in lines if not l.endswith(":")]
    labels, k = {}, 0
    for l in lines:
        if l.endswith(":"):
            labels[l[:-1]] = k
        else:
            k += 1
    return lds_loads_with_pending_lds_ops(body, labels)


def test_checker_flags_a_refill_after_an_unwaited_read():
    assert _check("""
        ds_read_b128 v[0:3], v4
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
    """) == [1]


def test_checker_accepts_a_refill_after_lgkmcnt0():
    assert _check("""
        ds_read_b128 v[0:3], v4
        s_waitcnt vmcnt(3) lgkmcnt(0)
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
    """) == []


def test_checker_follows_loops():
    assert _check("""
        .LBB0_1:
        buffer_load_dwordx4 v1, s[0:3], s4 offen lds
        ds_read_b128 v[0:3], v4
        s_cbranch_scc1 .LBB0_1
        s_endpgm
    """) == [0]
