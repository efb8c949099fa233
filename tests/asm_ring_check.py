"""Static check of register rings filled by inline-assembly loads.

A kernel may issue global loads as inline assembly and wait for them later
with an explicit `s_waitcnt vmcnt(N)`, so that several loads stay in flight in
registers.  The compiler takes such a load's destination as written when the
instruction issues; if it then copies, reuses or spills that register before
the wait (for instance a copy on a loop's back edge that it failed to
coalesce), the copy reads stale data and the load later lands in a register
that may hold something else.

This module reads the AMDGPU assembly of a kernel and follows every path of
its control-flow graph.  It tracks the destination registers of the
inline-assembly loads, each with the number of vector-memory instructions
issued after it, retires them at `s_waitcnt vmcnt(N)` once N or more younger
vector-memory instructions exist on every path, and reports any other
instruction that reads or writes a register still in flight.
"""
import re
import subprocess

_MEM_PREFIXES = ("global_", "buffer_", "flat_", "scratch_")
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_CAP = 64


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def kernel_bodies(asm):
    """{symbol: [lines]} for every kernel in an assembly file."""
    bodies = {}
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@", asm, re.M):
        start = m.end()
        end = re.compile(r"^\.Lfunc_end\d+:", re.M).search(asm, start).start()
        bodies[m.group(1)] = asm[start:end].split("\n")
    return bodies


def _blocks(lines):
    """Basic blocks: (label, [(text, in_asm)], successors)."""
    blocks = []
    cur = {"label": "__entry", "ins": []}
    in_asm = False
    for raw in lines:
        t = raw.split(";")[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t:
            continue
        if t.endswith(":") and not t.startswith("s_") and not t.startswith("v_"):
            blocks.append(cur)
            cur = {"label": t[:-1], "ins": []}
            continue
        if t.startswith("."):
            continue  # directives
        cur["ins"].append((t, in_asm))
    blocks.append(cur)
    labels = {b["label"]: i for i, b in enumerate(blocks)}
    for i, b in enumerate(blocks):
        succ = []
        falls = True
        for t, _ in b["ins"]:
            op = t.split()[0]
            if op == "s_branch":
                succ.append(labels[t.split()[1]])
                falls = False
            elif op.startswith("s_cbranch"):
                succ.append(labels[t.split()[1]])
            elif op in ("s_endpgm", "s_setpc_b64"):
                falls = False
        if falls and i + 1 < len(blocks):
            succ.append(i + 1)
        b["succ"] = succ
    return blocks


def _vmcnt(t):
    m = re.search(r"vmcnt\((\d+)\)", t)
    return int(m.group(1)) if m else None


def check(lines):
    """Hazards [(block label, instruction, registers)] of one kernel body."""
    blocks = _blocks(lines)
    state_in = [None] * len(blocks)
    state_in[0] = {}
    hazards = set()
    work = [0]
    while work:
        i = work.pop()
        st = dict(state_in[i])
        for t, in_asm in blocks[i]["ins"]:
            op = t.split()[0]
            args = t[len(op):]
            if op == "s_waitcnt":
                n = _vmcnt(t)
                if n is not None:
                    st = {r: p for r, p in st.items() if p < n}
                continue
            is_mem = op.startswith(_MEM_PREFIXES)
            used = _regs(args)
            clash = used & set(st)
            if clash:
                hazards.add((blocks[i]["label"], t, tuple(sorted(clash))))
            if is_mem:
                st = {r: min(p + 1, _CAP) for r, p in st.items()}
                if in_asm and "_load" in op and "_lds" not in op:
                    dst = t[len(op):].split(",")[0]
                    for r in _regs(dst):
                        st[r] = 0
        for j in blocks[i]["succ"]:
            old = state_in[j]
            if old is None:
                new = dict(st)
            else:
                new = dict(old)
                for r, p in st.items():
                    new[r] = min(p, new.get(r, _CAP)) if r in new else p
            if new != old:
                state_in[j] = new
                work.append(j)
    return sorted(hazards)


def compile_asm(hipcc, flags, src, out):
    subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", out], check=True,
                   capture_output=True, text=True)
    with open(out) as f:
        return f.read()
