"""Checks on the gfx950 assembly of the library's own kernels (test support).

`load_hazards` is a control-flow-aware pass over one kernel's instructions:
a VGPR that a global load writes may not be read or written again until an
s_waitcnt vmcnt retires that load on every path.  Each pending load carries
the minimum, over incoming paths, of the number of loads issued after it;
vmcnt(N) retires the loads whose minimum is at least N.  Loads into LDS
(global_load_lds_*) write no VGPR but still count.
"""

import re


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def kernels(asm_text, name_pattern):
    """(mangled name, body lines) of every kernel whose name matches."""
    out = []
    for m in re.finditer(r"^(_Z\S*" + name_pattern + r"\S*):[^\n]*\n(.*?)^\.Lfunc_end",
                         asm_text, re.S | re.M):
        out.append((m.group(1), m.group(2).splitlines()))
    return out


def metadata(asm_text):
    """name -> dict of the kernel descriptor fields we check."""
    meta = {}
    m = re.search(r"amdhsa\.kernels:(.*?)(?:\n\S|\Z)", asm_text, re.S)
    section = m.group(1) if m else asm_text
    for entry in re.split(r"\n  - ", section):
        nm = re.search(r"\.name:\s+(\S+)", entry)
        if not nm:
            continue
        def get(key, body=entry):
            g = re.search(r"\." + key + r":\s+(\S+)", body)
            return int(g.group(1)) if g else None
        meta[nm.group(1)] = {"private_segment_fixed_size": get("private_segment_fixed_size"),
                             "group_segment_fixed_size": get("group_segment_fixed_size"),
                             "vgpr_spill_count": get("vgpr_spill_count"),
                             "vgpr_count": get("vgpr_count")}
    return meta


def load_hazards(body_lines):
    instrs = [ln.split(";")[0].strip() for ln in body_lines]
    instrs = [t for t in instrs if t] + ["s_endpgm"]
    blocks, cur = [], []
    for t in instrs:
        if t.endswith(":"):
            if cur:
                blocks.append(cur)
            cur = [t]
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    labels = {b[0][:-1]: i for i, b in enumerate(blocks) if b[0].endswith(":")}
    succ = []
    for bi, b in enumerate(blocks):
        last = b[-1]
        if last.startswith("s_branch"):
            s = [labels[last.split()[1]]]
        elif last.startswith("s_cbranch"):
            s = [labels[last.split()[1]], bi + 1]
        elif last.startswith("s_endpgm"):
            s = []
        else:
            s = [bi + 1]
        succ.append([x for x in s if x < len(blocks)])
    state_in = [None] * len(blocks)
    state_in[0] = {}
    work, problems = [0], set()
    while work:
        bi = work.pop()
        st = dict(state_in[bi])
        for ii, t in enumerate(blocks[bi]):
            if t.endswith(":"):
                continue
            parts = re.split(r"[\s,]+", t)
            op = parts[0]
            if op == "s_waitcnt" and "vmcnt" in t:
                n = int(re.search(r"vmcnt\((\d+)\)", t).group(1))
                st = {k: v for k, v in st.items() if v[1] < n}
                continue
            if op.startswith(("global_load", "buffer_load", "scratch_load")):
                lds = "lds" in op
                dst = frozenset() if lds else _regs(parts[1])
                srcs = frozenset().union(*[_regs(p) for p in parts[(1 if lds else 2):]])
                if any(r & (dst | srcs) for r, _ in st.values()):
                    problems.add(t)
                st = {k: (r, a + 1) for k, (r, a) in st.items()}
                st[(bi, ii)] = (dst, 0)
                continue
            if op.startswith("s_"):
                continue
            used = frozenset().union(*[_regs(p) for p in parts[1:]])
            if any(r & used for r, _ in st.values()):
                problems.add(t)
        for s2 in succ[bi]:
            old = state_in[s2]
            if old is None:
                new = dict(st)
            else:
                new = dict(old)
                for k, (r, a) in st.items():
                    new[k] = (r, min(a, new[k][1])) if k in new else (r, a)
            if new != old:
                state_in[s2] = new
                work.append(s2)
    return sorted(problems)
