"""Static check of the gfx950 assembly of the attention kernels: distance in issue slots
between each matrix instruction and the first later instruction that touches its result.

The scaled FP8 matrix instruction used by the kernels (32x32x64, FP8 operands) needs 20 issue
slots before a vector instruction may read or overwrite its destination registers.  The
compiler pads for this itself, but one build of the backward kernel read the last accumulator
register after 19 slots filled with scalar instructions and produced wrong values in exactly
the rows that register holds.  This check walks every control path from each matrix
instruction (an s_nop N counts N + 1 slots, every other instruction one) and reports the
reads that come sooner.  A later matrix instruction that accumulates into exactly the same
registers is interlocked by the hardware and is not a read in this sense.
"""
import os
import re
import subprocess

NEED = 20


def compile_to_asm(src, out, hipcc, flags):
    """Device-only assembly of one HIP source with the library's own flags."""
    fl = [f for f in flags if f not in ("-shared", "-fPIC")]
    cmd = [hipcc] + fl + ["--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, res.stderr[-4000:]))
    return open(out).read()


def _regs(tok):
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instructions(asm, symbol):
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    ins = []
    for l in lines[start + 1:end]:
        t = l.split(";")[0].strip()
        if t.endswith(":"):
            ins.append(("LABEL", [t[:-1]]))
            continue
        if not t or t.startswith("."):
            continue
        parts = t.split(None, 1)
        ins.append((parts[0], re.split(r",\s*", parts[1]) if len(parts) > 1 else []))
    return ins


def _slots(op, ops):
    if op == "LABEL":
        return 0
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def kernel_symbols(asm, pattern):
    return sorted(set(re.findall(r"^(%s):" % pattern, asm, flags=re.M)))


def close_reads(asm, symbol, need=NEED):
    """[(index of matrix instruction, slots, reader)] for every read closer than `need`."""
    ins = _instructions(asm, symbol)
    labels = {ops[0]: i for i, (op, ops) in enumerate(ins) if op == "LABEL"}

    def successors(j):
        op, ops = ins[j]
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
        if op == "s_branch":
            return [labels[ops[0]]]
        nxt = [j + 1]
        if op.startswith("s_cbranch"):
            nxt.append(labels[ops[0]])
        return nxt

    found = []
    n_mfma = 0
    for i, (op, ops) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        n_mfma += 1
        dst = _regs(ops[0])
        best = None
        seen = {}
        stack = [(i + 1, 0)]
        while stack:
            j, w = stack.pop()
            if w >= need or j >= len(ins) or seen.get(j, need) <= w:
                continue
            seen[j] = w
            op2, ops2 = ins[j]
            if op2.startswith("v_mfma"):
                ab = _regs(ops2[1]) | _regs(ops2[2])
                c = _regs(ops2[3])
                hit = bool(ab & dst) or (bool(c & dst) and c != dst) or bool(_regs(ops2[0]) & dst and c != dst)
            elif op2 == "LABEL":
                hit = False
            else:
                touched = set()
                for o in ops2:
                    touched |= _regs(o)
                hit = bool(touched & dst)
            if hit:
                if best is None or w < best[0]:
                    best = (w, "%s %s" % (op2, ", ".join(ops2)))
                continue
            for s in successors(j):
                stack.append((s, w + _slots(op2, ops2)))
        if best is not None:
            found.append((i, best[0], best[1]))
    return found, n_mfma


def m0_uses(asm, symbol):
    """Instructions of `symbol` that read or write M0, as (index, text).  The kernels set M0 only
    for their direct global-to-LDS loads, in the fixed sequence s_mov_b32 m0 / s_nop 0 /
    global_load_lds_*; anything else touching M0 would be the compiler's, and could be clobbered
    by that sequence (the inline assembly's M0 clobber is not honoured: M0 is reserved)."""
    ins = _instructions(asm, symbol)
    out = []
    for i, (op, ops) in enumerate(ins):
        if op == "LABEL":
            continue
        if any(o.strip().split()[0] == "m0" for o in ops if o.strip()) or op.startswith("global_load_lds"):
            out.append((i, op, ops))
    return ins, out


def stray_m0_uses(asm, symbol):
    """M0 uses outside the direct-load sequence: [] when the kernel is safe."""
    ins, uses = m0_uses(asm, symbol)
    bad = []
    k = 0
    while k < len(uses):
        i, op, ops = uses[k]
        ok = (op == "s_mov_b32" and ops[0].strip() == "m0" and i + 2 < len(ins)
              and ins[i + 1][0] == "s_nop" and ins[i + 2][0].startswith("global_load_lds")
              and k + 1 < len(uses) and uses[k + 1][0] == i + 2)
        if ok:
            k += 2
            continue
        bad.append("%s %s" % (op, ", ".join(ops)))
        k += 1
    return bad
