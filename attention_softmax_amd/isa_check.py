"""Check gfx950 device assembly for reads of a matrix-core result that come too
soon after the MFMA instruction writing it.

An MFMA writes its destination registers over several passes, and CDNA3/CDNA4
do not interlock a later VALU, memory or LDS instruction that reads them: the
code must put enough independent instructions (wait states) in between. The
compiler inserts them, but it has been seen to miss the case where the read
sits at the head of a loop and the MFMA at the end of its previous iteration
(the read then sees a stale accumulator). This module walks every reading
instruction backwards through the instruction stream and through every branch
that reaches its block, and reports an MFMA destination read fewer than
``min_wait`` wait states later (``s_nop N`` counts N + 1; every other
instruction 1; an intervening write of the register ends the search).

    python -m attention_softmax_amd.isa_check file.s [...]

Used by the CPU tests on the attention sources as the build compiles them,
together with m0_outside_asm (no compiler use of m0 where inline assembly
sets it).
"""

import re
import sys

# A VALU read of an 8-pass XDL result needs 11 wait states on gfx950 (the
# 32x32x16 f16 / bf16 shapes used here are 8-pass).
MIN_WAIT = 11

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_STORES = ("global_store", "buffer_store", "ds_write", "ds_store", "flat_store", "scratch_store")
_NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), i) for i in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def parse(text):
    """{kernel symbol: [("label", name) | ("ins", text)]} of a .s file."""
    funcs, cur = {}, None
    for line in text.splitlines():
        if re.match(r"^_Z\w+:", line):
            cur = line.split(":")[0]
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if line.startswith("\t.section") or line.startswith(".Lfunc_end"):
            cur = None
            continue
        s = line.split(";")[0].rstrip()
        if not s.strip() or s.startswith("\t."):
            continue
        if re.match(r"^\.LBB\w+:", s):
            funcs[cur].append(("label", s[:-1]))
        else:
            funcs[cur].append(("ins", s.strip()))
    return funcs


def _wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _reads_writes(ins):
    """(registers read, registers written) of a non-MFMA instruction."""
    parts = ins.split(None, 1)
    if len(parts) < 2 or parts[0].startswith("s_"):
        return set(), set()
    ops = parts[1].split(",")
    if parts[0].startswith(_STORES):
        return _regs(parts[1]), set()
    return _regs(",".join(ops[1:])), _regs(ops[0])


def check_function(body, min_wait=MIN_WAIT):
    """[(reader instruction, MFMA instruction, wait states)] of one kernel."""
    labels = {x[1]: i for i, x in enumerate(body) if x[0] == "label"}
    preds = {}
    for i, (kind, s) in enumerate(body):
        if kind == "ins" and s.startswith(("s_branch", "s_cbranch")):
            target = s.split()[-1]
            if target in labels:
                preds.setdefault(labels[target], []).append(i)
    found = []

    def walk(i, need, dist, seen, reader):
        j = i - 1
        while j >= 0 and dist < min_wait:
            kind, s = body[j]
            if kind == "label":
                for p in preds.get(j, []):
                    if (p, j) not in seen:
                        walk(p + 1, need, dist, seen | {(p, j)}, reader)
                jj = j - 1
                while jj >= 0 and body[jj][0] == "label":
                    jj -= 1
                if jj >= 0 and body[jj][1].startswith(_NO_FALLTHROUGH):
                    return
                j -= 1
                continue
            if s.startswith("v_mfma"):
                if _regs(s.split(",")[0]) & need:
                    found.append((reader, s, dist))
                    return
            else:
                need = need - _reads_writes(s)[1]
                if not need:
                    return
            dist += _wait_states(s)
            j -= 1

    for i, (kind, s) in enumerate(body):
        if kind != "ins" or s.startswith("v_mfma"):
            continue
        reads = _reads_writes(s)[0]
        if reads:
            walk(i, reads, 0, frozenset(), s)
    return found


def check_text(text, min_wait=MIN_WAIT):
    """{kernel symbol: findings} for every kernel with a too-early read."""
    out = {}
    for name, body in parse(text).items():
        f = check_function(body, min_wait)
        if f:
            out[name] = f
    return out


def m0_outside_asm(text):
    """{kernel symbol: [instructions]} of compiler-emitted instructions that
    name m0, in kernels whose inline assembly sets m0 (the LDS loads issued
    from inline assembly there rely on the compiler keeping nothing in m0)."""
    out, cur, in_asm, sets, uses = {}, None, False, False, []
    def close():
        if cur is not None and sets and uses:
            out[cur] = uses
    for line in text.splitlines():
        if re.match(r"^_Z\w+:", line):
            close()
            cur, in_asm, sets, uses = line.split(":")[0], False, False, []
            continue
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        ins = s.split(";")[0].strip()
        if cur is None or not ins or not re.search(r"\bm0\b", ins):
            continue
        if in_asm:
            sets = True
        else:
            uses.append(ins)
    close()
    return out


def main(paths):
    bad = 0
    for path in paths:
        with open(path) as fh:
            res = check_text(fh.read())
        for name, found in res.items():
            bad += len(found)
            print(f"{path}: {name}: {len(found)} early read(s), e.g.")
            for reader, mfma, d in found[:3]:
                print(f"    {d} wait states: {mfma}  ->  {reader}")
    print(f"{bad} early read(s)")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
