"""Static checks of the generated assembly loops: the attention key loop and the projection's
reduction loop (test helper, no GPU).

Each loop is gfx950 assembly inside one inline-asm statement, so neither the compiler's hazard
recognizer nor its waitcnt insertion sees it.  This module re-checks what they would have:

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
  - LDS offsets stay inside the 128 KB the kernel allocates;
  - (projection) a scalar walk of the loop's control flow: every stage of the reduction is
    loaded once, complete, into the buffer it is read from, with the barriers that order the
    four wavefronts' loads and reads.
"""
from __future__ import annotations

import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_l1_amd", "csrc")

MFMA_WS = 12
LDS_BYTES = 131072


def load_generator(name="attn_loop_gen"):
    sys.path.insert(0, CSRC)
    try:
        import importlib
        mod = importlib.import_module(name)
    finally:
        sys.path.pop(0)
    return mod


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


def _call(gen, body, line):
    """The s_swappc line and the called routine."""
    p = parse(line)
    addr = int(re.search(r"s\[(\d+):", p[1][1]).group(1))
    if gen.FIXA <= addr < gen.FIXA + 8:
        k = (addr - gen.FIXA) // 2
        return [line] + routine(body, f".Lfix{k // 2}{k % 2}")
    k = (addr - gen.MASKA) // 2
    return [line] + routine(body, f".Lmask{k // 2}{k % 2}")


def expand(gen, lines, body, take_calls):
    """With take_calls (the taken path), follows every branch to an out-of-line call stub: the
    stub's call, the called routine, and the stub's branch back."""
    out = []
    for l in lines:
        out.append(l)
        p = parse(l)
        if take_calls and p and p[0] in ("s_cbranch_vccnz", "s_cbranch_scc1") and \
                p[1][0].endswith("_call"):
            stub = body.index(p[1][0] + ":")
            back = "s_branch " + p[1][0][:-5]
            j = stub + 1
            while body[j] != back:           # the stub: its tests, every call taken
                if body[j].startswith("s_swappc_b64"):
                    out.extend(_call(gen, body, body[j]))
                else:
                    out.append(body[j])
                j += 1
                assert j < len(body), f"malformed call stub {p[1][0]}"
            out.append(back)
        elif take_calls and p and p[0] == "s_swappc_b64":
            out.extend(_call(gen, body, l)[1:])
    return out


def traces(gen, checked=True):
    """(name, instruction list) for the paths through the loop: the prologue, n steps, the exit
    after the last one, with every call skipped or taken.  checked=False walks the fast body
    (its labels carry an F after .L, taken off here to match the step lists)."""
    body = [l.replace(".LF", ".L") for l in gen.generate(checked)]
    pro = gen.prologue(checked)
    steps = [gen.step(r, checked) for r in range(8)]
    epi = gen.epilogue(checked)
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


def check_hazards(gen, checked=True):
    errors = []
    for name, t in traces(gen, checked):
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


def check_registers(gen, hip_source, checked=True):
    decl = declared_registers(hip_source, gen)
    bad = set()
    for line in (gen.generate() if checked else gen.generate(False)):
        p = parse(line)
        if p is None:
            continue
        for o in p[1]:
            for r in regs(o):
                if r[0] in "vas" and r not in decl:
                    bad.add(f"{r} in: {line}")
    return sorted(bad)


def check_lds_bounds(gen, checked=True):
    """Largest byte an LDS read or a tile load can touch, over all lanes."""
    errors = []
    kmax = max(lq * 256 + 16 * (c ^ ((4 * (lq & 3)) + ((lq >> 2) & 3)))
               for lq in range(32) for c in range(16)) + 16
    vmax = 65536 + 15 * 256 + 16 * 15 + 8 + 8
    for line in (gen.generate() if checked else gen.generate(False)):
        m = re.search(r"offset:(\d+)", line)
        if line.startswith("ds_read_b128") and m and kmax + int(m.group(1)) > LDS_BYTES:
            errors.append(line)
        if line.startswith("ds_read_b64_tr_b16") and m and vmax + int(m.group(1)) > LDS_BYTES:
            errors.append(line)
        m0 = re.match(r"s_add_u32 m0, s\d+, (\d+)", line)
        if m0 and int(m0.group(1)) + 3 * 1024 + 1024 > LDS_BYTES:
            errors.append(line)
    return errors


# ------------------------------------------------------------------ the projection's loop

def proj_traces(gen, max_stages=5):
    """(name, instruction list): the prologue, n stages with the loop's exit test, the exit."""
    body = gen.generate()
    pro = body[:body.index(".Lploop:")]
    done = body[body.index(".Lpdone:") + 1:]
    tail = [f"s_add_u32 s{gen.STAGE}, s{gen.STAGE}, 1", f"s_cmp_eq_u32 s{gen.STAGE}, s{gen.NSTAGE}",
            "s_cbranch_scc1 .Lpdone"]
    for n in range(1, max_stages + 1):
        t = list(pro)
        for k in range(n):
            t += gen.stage(k % 2) + tail
        yield f"stages={n}", t + done


def check_proj_hazards(gen):
    errors = []
    for name, t in proj_traces(gen):
        c = Checker(name)
        c.run(t)
        errors += c.errors
    return errors


def check_proj_lds_bounds(gen, lds_bytes=LDS_BYTES):
    """Fragment reads: the address register of k-step u holds, per lane, row 128 w + lq of
    the X (or W) region, chunk (4u + g) ^ swizzle (w = 0, 1; lq < 16; g < 4); the immediate
    adds the buffer and 2048 bytes per row block.  Each read must stay inside the 32 KB half
    of the stage buffer its immediate names.  Tile loads: m0 immediate plus the wavefront's
    1 KB slot row."""
    errors = []
    span = max((w * 128 + lq) * 128 + 16 * ((4 * u + g) ^ (((w * 128 + lq) >> 1) & 7)) + 16
               for w in range(2) for lq in range(16) for u in range(2) for g in range(4))
    half = gen.XBUF[1] - gen.XBUF[0]
    for line in gen.generate():
        m = re.search(r"offset:(\d+)", line)
        if line.startswith("ds_read_b128") and m:
            addr = int(re.search(r"v(\d+) offset", line).group(1))
            off = int(m.group(1))
            is_w = gen.WADDR <= addr < gen.WADDR + 2
            base = gen.WBUF[0] if is_w else 0
            lo = base + off
            region = (gen.WBUF if is_w else gen.XBUF)[off // half]
            if lo + span > region + half or lo < region or lo + span > lds_bytes:
                errors.append(line)
        m0 = re.match(r"s_add_u32 m0, s\d+, (\d+)", line)
        if m0 and int(m0.group(1)) + 3 * 1024 + 1024 > lds_bytes:
            errors.append(line)
    return errors


def proj_stage_walk(gen, nstage, max_instructions=200000, rot=0):
    """Runs the generated loop's control flow for one wavefront with nstage stages, modelling
    the scalar registers it uses (stage counter, descriptor offset and range), the tile loads
    (which stage and which buffer part each fetches), vmcnt waits, barriers and fragment
    reads.  The tile starts at stage rot and wraps (its descriptors begin rot columns in).
    Returns (stages read per k-step, list of errors)."""
    body = [l for l in gen.generate() if not l.startswith(";")]
    labels = {l[:-1]: i for i, l in enumerate(body) if l.endswith(":")}
    sreg = {gen.NSTAGE: nstage, gen.WRAPT: nstage - rot, gen.WRAPB: nstage * 128}
    desc_off = {gen.XDESC: rot * 128, gen.WDESC: rot * 128}
    desc_live = {gen.XDESC: True, gen.WDESC: True}
    scc, m0, pc, steps = False, None, 0, 0
    inflight, content, errors, reads = [], {}, [], []
    last_read = {}          # buffer -> instruction count of the latest read
    barriers = []           # instruction counts of barriers
    landed = {}             # buffer -> instruction count of the wait that completed its last load
    stage_loads = {}
    val = lambda t: sreg.get(int(t[1:]), 0) if t.startswith("s") else int(t)
    while pc < len(body):
        steps += 1
        if steps > max_instructions:
            errors.append("no exit")
            break
        line = body[pc]
        pc += 1
        if line.endswith(":"):
            continue
        op, ops = parse(line)
        if op == "s_mov_b32" and ops[0] != "m0" and ops[1] != "m0":
            sreg[int(ops[0][1:])] = val(ops[1])
        elif op == "s_add_u32" and ops[0] == "m0":
            m0 = int(ops[2])
        elif op == "s_add_u32":
            d = int(ops[0][1:])
            if d in desc_off:
                desc_off[d] += val(ops[2])
            else:
                sreg[d] = val(ops[1]) + val(ops[2])
        elif op in ("s_cmp_ge_u32", "s_cmp_eq_u32"):
            x, y = val(ops[0]), val(ops[1])
            scc = x >= y if op == "s_cmp_ge_u32" else x == y
        elif op == "s_sub_u32":
            d = int(ops[0][1:])
            if d in desc_off:
                desc_off[d] -= val(ops[2])
            else:
                sreg[d] = val(ops[1]) - val(ops[2])
        elif op == "s_cselect_b32":
            d = int(ops[0][1:])
            if d - 2 in desc_live:
                if scc:
                    desc_live[d - 2] = False
            else:
                sreg[d] = val(ops[1]) if scc else val(ops[2])
        elif op == "s_cbranch_scc1":
            if scc:
                pc = labels[ops[0]]
        elif op == "s_branch":
            pc = labels[ops[0]]
        elif op == "s_barrier":
            barriers.append(steps)
        elif op == "buffer_load_dwordx4":
            d = int(re.match(r"s\[(\d+):", ops[1]).group(1))
            buf = (m0 % gen.WBUF[0]) // (gen.XBUF[1] - gen.XBUF[0])
            part = ("X" if d == gen.XDESC else "W", (m0 % (gen.XBUF[1] - gen.XBUF[0])) // gen.LOAD_BYTES)
            st = desc_off[d] // 128 if desc_live[d] else None
            if st is not None and not 0 <= desc_off[d] < nstage * 128:
                errors.append(f"load at column offset {desc_off[d]} outside the rows")
            if buf in last_read and not any(last_read[buf] < b for b in barriers):
                errors.append(f"load into buffer {buf} with no barrier after its last read")
            inflight.append((buf, part, st))
            if st is not None:
                stage_loads.setdefault(st, []).append((buf, part))
        elif op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", line)
            if m:
                while len(inflight) > int(m.group(1)):
                    buf, part, st = inflight.pop(0)
                    content.setdefault(buf, {})[part] = st
                    landed[buf] = steps
        elif op == "ds_read_b128":
            buf = int(re.search(r"offset:(\d+)", line).group(1)) // (gen.XBUF[1] - gen.XBUF[0])
            if any(b == buf for b, _, _ in inflight):
                errors.append(f"read of buffer {buf} while this wavefront still loads into it")
            got = set(content.get(buf, {}).values())
            if len(content.get(buf, {})) != 16 or len(got) != 1:
                errors.append(f"read of incomplete buffer {buf}: {content.get(buf)}")
            elif buf in landed and not any(landed[buf] < b for b in barriers):
                errors.append(f"read of buffer {buf} with no barrier after its loads landed")
            last_read[buf] = steps
            reads.append(got.pop() if len(got) == 1 else "?")
    if sreg.get(gen.STAGE) != nstage:
        errors.append(f"loop ended after {sreg.get(gen.STAGE)} stages, not {nstage}")
    for t in range(nstage):
        st = (rot + t) % nstage
        if sorted(stage_loads.get(st, [])) != sorted((t % 2, (x, i)) for x in "XW" for i in range(8)):
            errors.append(f"stage {st} loaded as {stage_loads.get(st)}")
    return [reads[i] for i in range(0, len(reads), gen.READS)], errors
