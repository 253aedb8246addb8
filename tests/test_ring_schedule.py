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
  its own path, not behind the wave's earlier reads of the slot it refills);
- the generated steady-state loop issues its loads in the order the counts
  assume, each wait at most its count (a hidden or scale load scheduled
  above a unit's direct load would make the count that retires that direct
  load one too large; the kernels fence their batches against it).
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


# The generated code issues the loads in the order the wait counts assume.
# The counts above are right for the source's issue order; the compiler must
# not move a load across one of the fenced waits. Along the steady-state loop
# of every instantiation, the sequence of vector memory loads and vmcnt waits
# must be one schedule period (or several) of the source, rotated to where
# the loop starts: per unit, a wait of at most the read's count; the unit's
# two direct loads, the hidden loads of a chunk's first unit, in the NVFP4
# kernel the two scale loads at a group's last chunk; at a chunk's last unit
# a wait of at most the hidden count. Extra waits, or waits of smaller
# counts, only wait longer and are accepted.

_VMCNT_RE = __import__("re").compile(r"vmcnt\((\d+)\)")
_BRANCH_RE = __import__("re").compile(r"^s_(?:cbranch_\w+|branch)\s+(\.LBB\S+)")
_SKINNY_RE = __import__("re").compile(r"skinny_kernelILi(\d+)ELi(\d+)ELb\dE\w+?Li(\d+)ELi(\d+)EE")
_NVRING_RE = __import__("re").compile(r"nvfp4_ring_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EE")


def _tokens(lines):
    out = []
    for t in lines:
        op = t.split()[0]
        if op.startswith("buffer_load"):
            out.append("D" if t.endswith(" lds") else "L")
        elif op.startswith(("global_load", "buffer_store", "global_store", "buffer_atomic")):
            out.append("X")  # no other vector memory operation belongs in the loop
        elif op == "s_waitcnt":
            m = _VMCNT_RE.search(t)
            if m:
                out.append(int(m.group(1)))
    return out


_HEADER_RE = __import__("re").compile(r"^(\.LBB\S+):\s*;\s*=>This Inner Loop Header", __import__("re").M)


def _main_loop(lines, labels, headers):
    """The loop (a header the compiler marks, to the last branch back to it)
    whose body holds the most direct loads: (start, end). Code laid out
    after a loop may branch back into it, so a backward branch alone does
    not make a loop."""
    best = None
    for i, t in enumerate(lines):
        m = _BRANCH_RE.match(t)
        if not m or m.group(1) not in headers or m.group(1) not in labels:
            continue
        j = labels[m.group(1)]
        if j <= i:
            n = sum(1 for k in range(j, i + 1) if lines[k].startswith("buffer_load") and lines[k].endswith(" lds"))
            if best is None or n > best[0] or (n == best[0] and i > best[2]):
                best = (n, j, i)
    assert best is not None and best[0] > 0
    return best[1], best[2]


def _model(kind, NB, NSL, HL, period, table):
    """One period of the source's loads and waits, unit by unit."""
    units = []
    for p in range(period):
        seq = [("W", table[p][0]), "D", "D"]
        if (p + NSL) % NB == 0:
            seq += ["L"] * HL
        if kind == "nvfp4" and (p // NB) % 8 == 7:
            seq += ["L", "L"]
        if p % NB == NB - 1:
            seq.append(("W", table[p][1]))
        units.append(seq)
    return units


def _gaps(seq, wait_of):
    """Loads in order and, per gap before each load, the vmcnt counts in it;
    the loop body is a cycle, so the gap after the last load joins the first."""
    loads, gaps, cur = [], [], []
    for t in seq:
        w = wait_of(t)
        if w is None:
            loads.append(t)
            gaps.append(cur)
            cur = []
        else:
            cur.append(w)
    if gaps:
        gaps[0] = cur + gaps[0]
    return loads, gaps


def _matches(asm, model):
    """asm (loads and vmcnt counts) against the model (loads and ("W", max)):
    the same loads in the same order, and in each gap between two loads the
    smallest asm count at most the smallest count the model needs there
    (waits between the same two loads act as their minimum)."""
    al, ag = _gaps(asm, lambda t: t if isinstance(t, int) else None)
    ml, mg = _gaps(model, lambda t: t[1] if isinstance(t, tuple) else None)
    if al != ml:
        return False
    return all(not m or (a and min(a) <= min(m)) for a, m in zip(ag, mg))


def _loop_follows_schedule(kind, NB, NSL, HL, period, table, lines, labels, headers):
    j, i = _main_loop(lines, labels, headers)
    asm = _tokens(lines[j:i + 1])
    if "X" in asm:
        return False
    units = _model(kind, NB, NSL, HL, period, table)
    n_dma = asm.count("D")
    if n_dma % (2 * period):
        return False
    reps = n_dma // (2 * period)
    for rot in range(period):
        flat = [t for u in (units[rot:] + units[:rot]) * reps for t in u]
        if _matches(asm, flat):
            return True
    return False


def test_generated_loop_issues_loads_in_schedule_order(ring_asm, schedules):
    kernels = kernel_bodies(ring_asm)
    checked, bad = 0, []
    for name, (lines, labels) in kernels.items():
        # label numbers restart in each compiled file: headers per kernel
        start = ring_asm.index("\n" + name + ":")
        headers = set(_HEADER_RE.findall(ring_asm[start:ring_asm.index(".Lfunc_end", start)]))
        m = _SKINNY_RE.search(name)
        if m:
            R, NB, NW, NSL = (int(x) for x in m.groups())
            kind, HL = "bf16", -(-16 * R * 8 // (64 * NW))
        else:
            m = _NVRING_RE.search(name)
            if not m:
                continue
            R, NB, NW, NSL = (int(x) for x in m.groups())
            kind, HL = "nvfp4", -(-16 * R * 32 // (64 * NW))
        assert (kind, NB, NSL, HL) in schedules, (name, "instantiation missing from the lists above")
        period, table = schedules[(kind, NB, NSL, HL)]
        if not _loop_follows_schedule(kind, NB, NSL, HL, period, table, lines, labels, headers):
            j, i = _main_loop(lines, labels, headers)
            bad.append(f"{name} (NB {NB}, NSL {NSL}, HL {HL}): {_tokens(lines[j:i + 1])[:80]}")
        checked += 1
    assert not bad, "\n".join(bad)
    assert checked >= 60


def test_schedule_order_check_flags_a_moved_load():
    # one unit of the bf16 kernel (NB = 1, NSL = 4, HL = 1): wait 5, two
    # direct loads, one hidden load, wait for the hidden chunk
    # (the loop is a cycle: the trailing hidden wait shares a gap with the
    # next unit's leading wait)
    model = [("W", 5), "D", "D", "L", ("W", 3)] * 2
    assert _matches([5, "D", "D", "L", 3, 5, "D", "D", "L", 3], model)
    assert _matches([4, 2, "D", "D", "L", 3, 3, "D", "D", "L", 2], model)  # extra, smaller waits
    # a load moved above the wait (where no other wait covers it)
    lead = [("W", 5), "D", "D", "L"] * 2
    assert _matches([5, "D", "D", "L", 5, "D", "D", "L"], lead)
    assert not _matches(["D", 5, "D", "L", 5, "D", "D", "L"], lead)
    # ... and covered by the previous iteration's trailing wait: accepted
    assert _matches(["D", 5, "D", "L", 3, "D", "D", "L", 3], model)
    assert not _matches([6, "D", "D", "L", 6, "D", "D", "L", 6], model)    # waits too weak
    assert not _matches([3, "D", "L", "D", 3, "D", "D", "L", 3], model)    # loads out of order
    assert not _matches([3, "D", "D", "L", 3, "D", "D", "L", "L"], model)  # a load too many
    assert not _matches([3, "D", "D", 3, "L", "D", "D", "L", 3], model)    # the hidden load late
