"""Static checks of the generated attention key loop (test helper, no GPU).

The loop is straight-line gfx950 assembly inside one inline-asm statement, so neither the
compiler's hazard recognizer nor its waitcnt insertion sees it.  This module re-checks what
they would have:

  - wait states (each instruction one, s_nop N = N + 1):
      MFMA result  -> any non-MFMA access       >= 12
      MFMA result  -> MFMA src A/B              >= 12   (src C of the same accumulator: 0)
      VALU write   -> MFMA read                 >= 2
      v_exp result -> VALU read                 >= 1
      v_dot2c      -> other read                >= 3
      m0 write     -> buffer load to LDS        >= 1
  - LDS results are used only after an lgkmcnt wait retires them, no register with an LDS
    result in flight is written, and at most 15 LDS operations are in flight;
  - every register the body touches is one of its operands or clobbers;
  - LDS offsets stay inside the 128 KB the kernel allocates.
"""
from __future__ import annotations

import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_l1_amd", "csrc")

MFMA_WS = 12
LDS_BYTES = 131072


def load_generator():
    sys.path.insert(0, CSRC)
    try:
        import attn_loop_gen
    finally:
        sys.path.pop(0)
    return attn_loop_gen


def regs(tok):
    tok = tok.strip()
    m = re.fullmatch(r"-?([vas])\[(\d+):(\d+)\]", tok)
    if m:
        return [(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    m = re.fullmatch(r"-?([vas])(\d+)", tok)
    if m:
        return [(m.group(1), int(m.group(2)))]
    if tok in ("vcc", "m0", "scc"):
        return [(tok, 0)]
    return []


def parse(line):
    line = line.split(";")[0].strip()
    if not line or line.endswith(":"):
        return None
    parts = line.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], [o.split()[0] if o else o for o in ops]


CONTROL = {"s_waitcnt", "s_barrier", "s_nop", "s_branch", "s_cbranch_scc1", "s_cbranch_scc0",
           "s_cbranch_vccz", "s_cbranch_vccnz", "s_swappc_b64", "s_setpc_b64", "s_getpc_b64"}


def classify(op, ops):
    """(kind, destination registers, source registers); MFMA sources split into A, B, C."""
    if op.startswith("v_mfma"):
        return "mfma", regs(ops[0]), {"A": regs(ops[1]), "B": regs(ops[2]), "C": regs(ops[3])}
    if op.startswith("ds_read") or op.startswith("ds_bpermute"):
        return "lds", regs(ops[0]), [r for o in ops[1:] for r in regs(o)]
    if op.startswith("buffer_load"):
        return "vmem_lds", [], [r for o in ops for r in regs(o)] + [("m0", 0)]
    if op in CONTROL:
        return "ctl", [], []
    kind = "salu" if op.startswith("s_") else "valu"
    if op.startswith("v_cmp") and not op.endswith("_e64"):
        return kind, [("vcc", 0)], [r for o in ops[1:] for r in regs(o)]
    if op == "v_dot2c_f32_bf16":
        return "dot", regs(ops[0]), regs(ops[0]) + [r for o in ops[1:] for r in regs(o)]
    if op == "v_exp_f32":
        kind = "trans"
    srcs = [r for o in ops[1:] for r in regs(o)]
    if op.startswith("v_cndmask") and "vcc" not in ops[1:]:
        srcs.append(("vcc", 0))
    if op in ("s_cselect_b32", "s_addc_u32"):
        srcs.append(("scc", 0))
    dsts = regs(ops[0]) if ops else []
    if op.startswith("s_add") or op.startswith("s_sub"):
        dsts = dsts + [("scc", 0)]
    if op.startswith("s_cmp"):
        dsts, srcs = [("scc", 0)], [r for o in ops for r in regs(o)]
    return kind, dsts, srcs


class Checker:
    def __init__(self, name):
        self.name, self.ws, self.n = name, 0, 0
        self.last = {}          # register -> (kind, wait-state clock at issue, destination tuple)
        self.lds = []           # LDS operations in flight: their destination registers
        self.errors = []

    def err(self, msg, line):
        self.errors.append(f"[{self.name} #{self.n}] {msg}: {line}")

    def run(self, lines):
        for line in lines:
            p = parse(line)
            if p is None:
                continue
            self.n += 1
            op, ops = p
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", line)
                if m:
                    while len(self.lds) > int(m.group(1)):
                        self.lds.pop(0)
            kind, dsts, srcs = classify(op, ops)
            allsrc = srcs if isinstance(srcs, list) else srcs["A"] + srcs["B"] + srcs["C"]
            for r in allsrc + dsts:
                if any(r in pend for pend in self.lds):
                    self.err(f"{r} used or overwritten while an LDS result is in flight", line)
            for r in allsrc:
                if r not in self.last:
                    continue
                pk, pws, prange = self.last[r]
                dist, need = self.ws - pws, 0
                if pk == "mfma":
                    same_acc = kind == "mfma" and r in srcs["C"] and tuple(srcs["C"]) == prange
                    need = 0 if same_acc else MFMA_WS
                elif pk in ("valu", "trans", "dot") and kind == "mfma":
                    need = 2
                if pk == "trans" and kind in ("valu", "trans", "dot"):
                    need = max(need, 1)
                if pk == "dot" and kind != "dot":
                    need = max(need, 3)
                if pk == "salu" and r == ("m0", 0) and kind == "vmem_lds":
                    need = 1
                if dist < need:
                    self.err(f"{r} written by {pk} {dist} wait states earlier, needs {need}", line)
            for r in dsts:
                if r in self.last and self.last[r][0] == "mfma" and kind != "mfma":
                    if self.ws - self.last[r][1] < MFMA_WS:
                        self.err(f"{r} overwritten too soon after an MFMA wrote it", line)
            if kind == "lds":
                self.lds.append(set(dsts))
                if len(self.lds) > 15:
                    self.err("more than 15 LDS operations in flight", line)
            for r in dsts:
                self.last[r] = (kind, self.ws + 1, tuple(dsts))
            self.ws += int(ops[0], 0) + 1 if op == "s_nop" else 1


def routine(body, label):
    i = body.index(label + ":")
    out = []
    for l in body[i + 1:]:
        out.append(l)
        if l.startswith("s_setpc_b64"):
            return out
    raise ValueError(label)


def expand(gen, lines, body, take_calls):
    """Inlines the called routine after every s_swappc when take_calls (the taken path)."""
    out = []
    for l in lines:
        out.append(l)
        p = parse(l)
        if take_calls and p and p[0] == "s_swappc_b64":
            addr = int(re.search(r"s\[(\d+):", p[1][1]).group(1))
            if gen.FIXA <= addr < gen.FIXA + 8:
                k = (addr - gen.FIXA) // 2
                out.extend(routine(body, f".Lfix{k // 2}{k % 2}"))
            else:
                k = (addr - gen.MASKA) // 2
                out.extend(routine(body, f".Lmask{k // 2}{k % 2}"))
    return out


def traces(gen):
    """(name, instruction list) for the paths through the loop: the prologue, n steps, the exit
    after the last one, with every call skipped or taken."""
    body = gen.generate()
    pro = gen.prologue()
    steps = [gen.step(r) for r in range(8)]
    epi = gen.epilogue()
    exits = []
    for x in range(2):
        i = epi.index(f".Lexit{x}:")
        exits.append(epi[i + 1:epi.index("s_branch .Ldone", i)])
    done = body[body.index(".Ldone:") + 1:]
    for take in (False, True):
        for last in (6, 7, 12):
            t = list(pro)
            for k in range(last + 1):
                t += steps[k % 8]
            t += exits[((last % 8) & 1) ^ 1] + done
            yield f"calls={take} last_step={last}", expand(gen, t, body, take)


def check_hazards(gen):
    errors = []
    for name, t in traces(gen):
        c = Checker(name)
        c.run(t)
        errors += c.errors
    return errors


def declared_registers(hip_source, gen):
    """Registers named by the asm statement's operand constraints plus its clobber list."""
    decl = set()
    for m in re.finditer(r'"[+=]?\{([vas])\[(\d+):(\d+)\]\}"', hip_source):
        decl |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r'"[+=]?\{([vas])(\d+)\}"', hip_source):
        decl.add((m.group(1), int(m.group(2))))
    for kind, s in gen.clobbered().items():
        decl |= {(kind, i) for i in s}
    return decl


def check_registers(gen, hip_source):
    decl = declared_registers(hip_source, gen)
    bad = set()
    for line in gen.generate():
        p = parse(line)
        if p is None:
            continue
        for o in p[1]:
            for r in regs(o):
                if r[0] in "vas" and r not in decl:
                    bad.add(f"{r} in: {line}")
    return sorted(bad)


def check_lds_bounds(gen):
    """Largest byte an LDS read or a tile load can touch, over all lanes."""
    errors = []
    kmax = max(lq * 256 + 16 * (c ^ ((4 * (lq & 3)) + ((lq >> 2) & 3)))
               for lq in range(32) for c in range(16)) + 16
    vmax = 65536 + 15 * 256 + 16 * 15 + 8 + 8
    for line in gen.generate():
        m = re.search(r"offset:(\d+)", line)
        if line.startswith("ds_read_b128") and m and kmax + int(m.group(1)) > LDS_BYTES:
            errors.append(line)
        if line.startswith("ds_read_b64_tr_b16") and m and vmax + int(m.group(1)) > LDS_BYTES:
            errors.append(line)
        m0 = re.match(r"s_add_u32 m0, s\d+, (\d+)", line)
        if m0 and int(m0.group(1)) + 3 * 1024 + 1024 > LDS_BYTES:
            errors.append(line)
    return errors
