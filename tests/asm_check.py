"""Checks on the gfx950 assembly of this library's own kernels (test helper).

A direct-to-LDS load (`buffer_load_* ... lds`) writes LDS, but its completion
is counted by vmcnt, not lgkmcnt. In a kernel whose waves share a stage that
such loads fill, every `s_barrier` that hands the stage over must come after a
`s_waitcnt vmcnt(k)` that retires those loads: vector memory loads complete in
issue order, so vmcnt(k) retires every load issued before the last k.
"""
import re

_LABEL = re.compile(r"^(\.LBB\S+):")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")


def kernel_bodies(asm: str):
    """{symbol: [instruction, ...]} plus the label map, for every kernel in `asm`."""
    out = {}
    for m in re.finditer(r"\n(_Z[^:\s]+):", asm):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        if end < 0:
            continue
        lines, labels = [], {}
        for raw in asm[m.end():end].split("\n"):
            t = raw.split(";")[0].strip()
            lm = _LABEL.match(t)
            if lm:
                labels[lm.group(1)] = len(lines)
                continue
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            lines.append(t)
        out[name] = (lines, labels)
    return out


def barriers_with_pending_lds_loads(lines, labels):
    """Indices of `s_barrier`s reached on some path with a direct-to-LDS load
    possibly outstanding.

    State along a path: 0 = none outstanding; n > 0 = the youngest direct load
    is followed by n - 1 later vector memory instructions. A waitcnt
    vmcnt(k) with k < n retires it. Paths are followed through every branch
    (a worklist over (instruction, state)), so loops are covered."""
    bad = set()
    best = {}
    work = [(0, 0)]
    while work:
        p, st = work.pop()
        while p < len(lines):
            if best.get(p, -1) >= st:
                break
            best[p] = st
            t = lines[p]
            op = t.split()[0]
            if op.startswith("buffer_load") and t.endswith(" lds"):
                st = 1
            elif (op.startswith("buffer_") or op.startswith("global_")) and st:
                st = min(st + 1, 64)
            if op == "s_waitcnt":
                w = _VMCNT.search(t)
                if w and st and int(w.group(1)) < st:
                    st = 0
            if op == "s_barrier" and st:
                bad.add(p)
            if op == "s_branch" or op.startswith("s_cbranch"):
                tgt = t.split()[1]
                if tgt in labels:
                    work.append((labels[tgt], st))
                if op == "s_branch":
                    break
            if op == "s_endpgm":
                break
            p += 1
    return sorted(bad)


_LGKM0 = re.compile(r"lgkmcnt\(0\)")


def lds_loads_with_pending_lds_ops(lines, labels):
    """Indices of direct-to-LDS loads reached on some path while an LDS
    instruction of the same wave (a `ds_` read, write or permute) may still
    be outstanding.

    A direct-to-LDS load writes LDS on its own path, not behind the wave's
    earlier LDS instructions, so a ring kernel that refills a slot it has
    just read must first wait for those reads (`s_waitcnt lgkmcnt(0)`).
    State along a path: whether a `ds_` instruction was issued since the
    last lgkmcnt(0); followed through every branch, as above."""
    bad = set()
    best = {}
    work = [(0, 0)]
    while work:
        p, st = work.pop()
        while p < len(lines):
            if best.get(p, -1) >= st:
                break
            best[p] = st
            t = lines[p]
            op = t.split()[0]
            if op.startswith("ds_"):
                st = 1
            if op == "s_waitcnt" and _LGKM0.search(t):
                st = 0
            if op.startswith("buffer_load") and t.endswith(" lds") and st:
                bad.add(p)
            if op == "s_branch" or op.startswith("s_cbranch"):
                tgt = t.split()[1]
                if tgt in labels:
                    work.append((labels[tgt], st))
                if op == "s_branch":
                    break
            if op == "s_endpgm":
                break
            p += 1
    return sorted(bad)
