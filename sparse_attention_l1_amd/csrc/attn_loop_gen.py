"""Generates the key loop of the D = 128 attention kernel (attn_pipe.hip) as gfx950 assembly.

Active-query full-context attention ("Technische Samenvatting: Heterogene Staptoewijzing (HSA)
voor Efficiënte Videogeneratie", §2.2 items 3-4): the active queries of one (b, h) attend to all
N cached keys, O = softmax(Q_A K^T * scale) V.  The method is the one of attn.hip's kernel
(transposed MFMAs, base-2 online softmax against a reference max, a rare path that takes the
true max when a block's sum exceeds 2^8 or is not a number); only the row sums differ (below).  This file
fixes the order in which one wavefront issues the work, which the compiler does not find.

Why hand scheduled.  One wavefront per SIMD owns 64 queries (two 32-query blocks qb = 0, 1),
so each K/V fragment read from LDS feeds two MFMAs and the O accumulators (128 AGPRs) and the
Q^T fragments (64 AGPRs) stay in the accumulation registers.  With a single wave per SIMD the
VALU work of the softmax (about as many issue cycles as the MFMAs leave free) only overlaps the
matrix cores if it is spread evenly between the MFMAs of the same wave.

Key blocks are 32 keys (block x).  Step s of the loop has two halves of 16 MFMA slots:

  H1(s): the S^T chains S(s+1, 1) and S(s+2, 0), interleaved (two independent accumulators)
         VALU: pairs 4..7 of softmax(s+1, 0) and softmax(s, 1), then their range checks
         LDS:  the 16 transposing reads of V(s+1)
  H2(s): the P.V groups PV(s, 1) and PV(s+1, 0), interleaved
         VALU: pairs 0..3 of softmax(s+1, 1) and softmax(s+2, 0) (after the ragged-block masks)
         LDS:  the 8 fragment reads of K(s+3)

so every softmax spreads over one full step and no slot holds more VALU work than another.
Buffers: S, P, K fragments and V fragments are double buffered by block parity.  Tiles of 4
blocks travel global -> LDS by buffer loads with an LDS destination (rows past the key count
are out of the descriptor's range and read as zero); V tile j holds blocks 4j..4j+3, K tile j
blocks 4j+2..4j+5, and one barrier every 4 steps (s = 3 mod 4) refills the two buffers freed
since the last one.  The loop body is unrolled over 8 steps so that every LDS offset is an
immediate.  The rare-path and ragged-block routines are called from stubs out of line, so
each step's four tests fall through branches that are not taken.

Row sums: the normaliser of a query is the sum of the bf16-rounded P that the P.V MFMAs
consume, so a key that dominates the softmax is weighted by exactly p / sum(p) whatever the
rounding of p.  After each pair is rounded into its packed register, the two bf16 halves are
read back as fp32 (the high half by masking off the low 16 bits, the low half by a 16-bit left
shift) and added; the four pair sums of a half block are added as a tree, (ps0 + ps1) +
(ps2 + ps3), into this lane's block sum.  A lane holds 16 of a query's 32 keys per block, so
the running sum is per lane; the two lanes of a query add theirs at the end.  (Row sums by
16x16x32 or 4x4x4 MFMAs on the packed P, with a 0/1 operand, cost 11-19% of the kernel's time:
more than these 24 extra VALU instructions per block.)

Two bodies: generate(True) is the checked loop described above; generate(False) is the fast
loop, which sets each query block's reference max from key block 0 in the prologue and then
drops every range check (the block sums only go into L) and the ragged-block masks, so no
step has a data-dependent branch or a test.  Its keys past the end of the last block keep
s = 0 (their K and V rows read as zero), so each adds exactly bf16(2^-m) to the row sum and
nothing to O; the kernel subtracts that from L afterwards.  Its labels carry an F after .L so that both bodies can sit in one kernel; the kernel
runs the checked body only for workgroups with a query whose fast row sum left [1, 2^64].

Register map (per lane):  VGPR  S 0-63, P 64-95, K fragments 96-159, LDS/buffer addresses
160-183, softmax state 184-194, temps 196-218;  AGPR  O 0-127, Q^T 128-191, V^T fragments
192-255;  SGPR 40-77 (descriptors, counters, routine addresses).
"""
import re
import sys

# ---------------------------------------------------------------- register map
def S(par, qb):            # S^T accumulator (32 keys x 32 queries): 16 VGPRs
    return 0 + (par * 2 + qb) * 16
def P(par, qb):            # P^T as bf16 pairs: 8 VGPRs, reg t = keys 2t, 2t+1 of the lane's run
    return 64 + (par * 2 + qb) * 8
def KF(par, u):            # K fragment u of one block (A operand of the S MFMA): 4 VGPRs
    return 96 + par * 32 + u * 4
KADDR = 160                # 8: LDS byte address of K fragment u (block 0 of buffer 0)
VADDR = 168                # 8: [hh*4 + e] LDS byte address of a V transposing read
VOFF = 176                 # 8: buffer offset of tile-load instruction i
M = 184                    # +qb reference max (log2 units)
L = 186                    # +qb running sum of the rounded P (this lane's half of the keys)
NEGM = 188                 # +qb  -M
VAX = 190                  # (lane ^ 32) * 4, ds_bpermute address of the partner lane
VT = 191                   # 4*g - lim for the ragged last block
VNINF = 192                # -inf
LS = 193                   # +qb block sum (this lane's 16 keys)
def TMP(qb):               # 8 softmax temps (4 pairs in flight) per query block
    return 196 + qb * 9
T0 = 214                   # rare-path temps T0..T0+4
NV_END = 219

def O(qb, e):              # O^T accumulator (AGPR), 16 regs
    return (qb * 4 + e) * 16
def Q(qb, u):              # Q^T fragment (AGPR), 4 regs
    return 128 + (qb * 8 + u) * 4
def VF(par, e, h2):        # V^T fragment (AGPR), 4 regs: [hh = 0: 2 regs, hh = 1: 2 regs]
    return 192 + par * 32 + (e * 2 + h2) * 4

# SGPRs
KDESC = 40                 # s[40:43] buffer descriptor of the K slice (advances per tile)
VDESC = 44                 # s[44:47] same for V
SC = 48                    # scale * log2(e)
STEP = 49
LAST = 50                  # index of the last step (n_blocks - 2)
MASK1 = 51                 # step whose softmax(s+1, 1) is the ragged last block, else -1
M0SAVE = 52
M0BASE = 53                # LDS base + wave * 1024
ADV = 54                   # bytes per tile of 128 rows
NINF = 55
FIXA = 56                  # 4 x 2: rare-path routine addresses [par*2 + qb]
MASKA = 64                 # 4 x 2: mask routine addresses
RET = 72
STMP = 74
MASK0 = 76                 # step whose softmax(s+2, 0) is the ragged last block, else -1

KBUF = 0                   # LDS byte offset of the two K tile buffers (32 KB each)
VBUF = 65536               # V tile buffers
TILE_BYTES = 32768
BLK_BYTES = 8192           # 32 keys x 256 B

# Inputs the kernel passes in pinned registers (operand constraints of the asm statement).
PINNED_IN = {"v": set(range(160, 192)), "a": set(range(0, 192)),
             "s": {KDESC + i for i in range(4)} | {VDESC + i for i in range(4)} |
                  {SC, LAST, MASK1, M0BASE, ADV}}


def v(r, n=1):
    return f"v{r}" if n == 1 else f"v[{r}:{r + n - 1}]"
def a(r, n=1):
    return f"a{r}" if n == 1 else f"a[{r}:{r + n - 1}]"
def s(r, n=1):
    return f"s{r}" if n == 1 else f"s[{r}:{r + n - 1}]"


# ---------------------------------------------------------------- instruction builders
def mfma_s(par, qb, u):
    """S^T(block of parity par, query block qb) += K fragment u . Q^T fragment u."""
    src_c = "0" if u == 0 else v(S(par, qb), 16)
    return (f"v_mfma_f32_32x32x16_bf16 {v(S(par, qb), 16)}, {v(KF(par, u), 4)}, "
            f"{a(Q(qb, u), 4)}, {src_c}")

def mfma_pv(par, qb, e, h2):
    """O^T(qb, rows 32e..32e+31) += V^T fragment (block parity par, e, key step h2) . P^T."""
    return (f"v_mfma_f32_32x32x16_bf16 {a(O(qb, e), 16)}, {a(VF(par, e, h2), 4)}, "
            f"{v(P(par, qb) + 4 * h2, 4)}, {a(O(qb, e), 16)}")

def kpos(x):
    """(buffer, position) of key block x among the K tiles (tile j = blocks 4j+2..4j+5)."""
    j = (x - 2) // 4
    return j & 1, (x - 2) % 4

def vpos(x):
    j = x // 4
    return j & 1, x % 4

def kread(x, u):
    tb, blk = kpos(x)
    return (f"ds_read_b128 {v(KF(x & 1, u), 4)}, {v(KADDR + u)} "
            f"offset:{KBUF + tb * TILE_BYTES + blk * BLK_BYTES}")

def vread(x, e, h2, hh):
    tb, blk = vpos(x)
    off = tb * TILE_BYTES + blk * BLK_BYTES + h2 * 4096      # VADDR includes VBUF
    return (f"ds_read_b64_tr_b16 {a(VF(x & 1, e, h2) + 2 * hh, 2)}, {v(VADDR + hh * 4 + e)} "
            f"offset:{off}")

def vreads(x):
    """The 16 transposing reads of block x, in the order the P.V MFMAs consume them."""
    return [vread(x, e, h2, hh) for h2 in range(2) for e in range(4) for hh in range(2)]

def tile_load_pairs(desc, buf_base, i_range):
    """(m0 write, load) pairs; load i of a wave fills rows 16i..16i+15 of the tile."""
    return [(f"s_add_u32 m0, {s(M0BASE)}, {buf_base + i * 4096}",
             f"buffer_load_dwordx4 {v(VOFF + i)}, {s(desc, 4)}, 0 offen lds") for i in i_range]

def desc_advance(desc):
    """Moves a descriptor one tile on; the remaining byte count saturates at zero."""
    return [f"s_add_u32 {s(desc)}, {s(desc)}, {s(ADV)}",
            f"s_addc_u32 {s(desc + 1)}, {s(desc + 1)}, 0",
            f"s_sub_u32 {s(desc + 2)}, {s(desc + 2)}, {s(ADV)}",
            f"s_cselect_b32 {s(desc + 2)}, 0, {s(desc + 2)}"]


def softmax_part(par, qb, t0, t1):
    """Pairs t0..t0+3 of one softmax block: x, y = 2^(s*c - m); P[t] = bf16(x, y); the two
    rounded halves of P[t] read back as fp32 and added (the pair sum of the values the MFMA
    uses); the four pair sums added as a tree into LS (set by the first half, added to by the
    second).  A pair's consumers come after the next pair's exponentials."""
    assert t1 == t0 + 4
    sb, pb, tmp = S(par, qb), P(par, qb), TMP(qb)
    ops = []
    def xy(t):
        return tmp + 2 * (t % 4), tmp + 2 * (t % 4) + 1
    def finish(t):
        x, y = xy(t)
        return [f"v_cvt_pk_bf16_f32 {v(pb + t)}, {v(x)}, {v(y)}",
                f"v_and_b32 {v(y)}, 0xffff0000, {v(pb + t)}",
                f"v_lshlrev_b32 {v(x)}, 16, {v(pb + t)}",
                f"v_add_f32 {v(x)}, {v(x)}, {v(y)}"]
    pend = None
    for t in range(t0, t1):
        x, y = xy(t)
        ops.append(f"v_fma_f32 {v(x)}, {v(sb + 2 * t)}, {s(SC)}, {v(NEGM + qb)}")
        ops.append(f"v_fma_f32 {v(y)}, {v(sb + 2 * t + 1)}, {s(SC)}, {v(NEGM + qb)}")
        ops.append(f"v_exp_f32 {v(x)}, {v(x)}")
        ops.append(f"v_exp_f32 {v(y)}, {v(y)}")
        if pend is not None:
            ops.extend(finish(pend))
        pend = t
    ops.extend(finish(pend))       # two instructions after the last exponential
    x0, x1, x2, x3 = (xy(t)[0] for t in range(t0, t1))
    ops.append(f"v_add_f32 {v(x0)}, {v(x0)}, {v(x1)}")
    ops.append(f"v_add_f32 {v(x2)}, {v(x2)}, {v(x3)}")
    if t0 == 0:
        ops.append(f"v_add_f32 {v(LS + qb)}, {v(x0)}, {v(x2)}")
    else:
        ops.append(f"v_add_f32 {v(x0)}, {v(x0)}, {v(x2)}")
        ops.append(f"v_add_f32 {v(LS + qb)}, {v(LS + qb)}, {v(x0)}")
    return ops


def softmax_full(par, qb):
    return softmax_part(par, qb, 0, 4) + softmax_part(par, qb, 4, 8)


# Calls of the rare-path and mask routines sit out of line, in stubs after the routines: the
# common case falls through a branch that is not taken (a taken branch refetches instructions,
# and with one wavefront per SIMD nothing else issues meanwhile).  The stub calls the routine
# and branches back to the label after the call site.
CALL_STUBS = {}            # call-site label -> the routine's address register pair


def call_site(branch, routine_regs, label):
    CALL_STUBS[label] = routine_regs
    return [f"{branch} {label}_call", f"{label}:"]


def call_stubs(body):
    """A stub calls its routine (or, for a pair check, each block's routine that its own range
    check asks for) and branches back."""
    out = []
    for l in body:
        if l.endswith("_call") and l.startswith("s_cbranch"):
            label = l.split()[1][:-len("_call")]
            stub = CALL_STUBS[label]
            if isinstance(stub, str):
                out += [f"{label}_call:", f"s_swappc_b64 {s(RET, 2)}, {stub}"]
            else:
                out.append(f"{label}_call:")
                for k, (qb, regs) in enumerate(stub):
                    out += [f"v_cmp_nge_f32 vcc, 0x43800000, {v(LS + qb)}",
                            f"s_cbranch_vccz {label}_n{k}",
                            f"s_swappc_b64 {s(RET, 2)}, {regs}",
                            f"{label}_n{k}:"]
            out.append(f"s_branch {label}")
    return out


def check_and_fix(par, qb, label):
    """Calls the rare path if any lane's block sum is not in (-inf, 256]; then L += LS."""
    return ([f"v_cmp_nge_f32 vcc, 0x43800000, {v(LS + qb)}"] +
            call_site("s_cbranch_vccnz", s(FIXA + 2 * (par * 2 + qb), 2), label) +
            [f"v_add_f32 {v(L + qb)}, {v(L + qb)}, {v(LS + qb)}"])


def check_pair_and_fix(blocks, label):
    """Range check of two blocks with one branch: the two lanes' block sums are added (a sum
    of non-negative values is in (-inf, 256] only if both are, and inf or NaN carries through),
    and only if some lane's total is out of range does the stub test the blocks one by one and
    call the rare path for each that needs it.  Then L += LS for both.  One data-dependent
    branch per step instead of two: the second one cost 7% of the loop (measured on MI355X)."""
    (pa, qa), (pb, qb) = blocks
    CALL_STUBS[label] = [(qa, s(FIXA + 2 * (pa * 2 + qa), 2)), (qb, s(FIXA + 2 * (pb * 2 + qb), 2))]
    return [f"v_add_f32 {v(T0)}, {v(LS + qa)}, {v(LS + qb)}",
            f"v_cmp_nge_f32 vcc, 0x43800000, {v(T0)}",
            f"s_cbranch_vccnz {label}_call", f"{label}:",
            f"v_add_f32 {v(L + qa)}, {v(L + qa)}, {v(LS + qa)}",
            f"v_add_f32 {v(L + qb)}, {v(L + qb)}, {v(LS + qb)}"]


def add_block_sums(*blocks):
    """L += LS for each (parity, query block) without a range check (the fast body)."""
    return [f"v_add_f32 {v(L + qb)}, {v(L + qb)}, {v(LS + qb)}" for _, qb in blocks]


def init_reference_max(par, qb):
    """Sets the reference max of query block qb to the true max of its S^T block (both lanes of a
    query), before any of that query's exponentials: the fast body never raises it in the
    loop, so every later p is 2^(c s - m) against this block's max."""
    sb = S(par, qb)
    t1, t3 = T0 + 1, T0 + 3
    out = [f"v_max3_f32 {v(t1)}, {v(sb)}, {s(NINF)}, {v(sb + 1)}"]
    for j in range(2, 16, 2):
        out.append(f"v_max3_f32 {v(t1)}, {v(t1)}, {v(sb + j)}, {v(sb + j + 1)}")
    out += ["s_waitcnt lgkmcnt(0)",
            f"ds_bpermute_b32 {v(t3)}, {v(VAX)}, {v(t1)}",
            "s_waitcnt lgkmcnt(0)",
            f"v_max_f32 {v(t3)}, {v(t1)}, {v(t3)}",
            f"v_mul_f32 {v(t3)}, {s(SC)}, {v(t3)}",
            f"v_mov_b32 {v(M + qb)}, {v(t3)}",
            f"v_xor_b32 {v(NEGM + qb)}, 0x80000000, {v(t3)}"]
    return out


def mask_call(par, qb, stepreg, label):
    return ([f"s_cmp_eq_u32 {s(STEP)}, {s(stepreg)}"] +
            call_site("s_cbranch_scc1", s(MASKA + 2 * (par * 2 + qb), 2), label))


def cost(op):
    """Issue weight of one instruction for the slot balance (a transcendental ~2.25 VALU)."""
    if op.startswith("v_exp"):
        return 2.25
    if op.startswith("v_"):
        return 1.0
    if op.startswith("s_nop"):
        return 0.25
    if op.startswith("s_"):
        return 0.5
    return 0.0


def merge(a_ops, b_ops):
    """Round-robin merge of two independent instruction lists (each keeps its order)."""
    out, i, j = [], 0, 0
    while i < len(a_ops) or j < len(b_ops):
        if i < len(a_ops):
            out.append(a_ops[i]); i += 1
        if j < len(b_ops):
            out.append(b_ops[j]); j += 1
    return out


def place(ops, slots):
    """Splits ops, in order, over the given MFMA slots with about equal issue weight each."""
    total = sum(cost(o) for o in ops)
    per = total / len(slots)
    res = {sl: [] for sl in slots}
    acc, k = 0.0, 0
    for o in ops:
        while k < len(slots) - 1 and acc >= per * (k + 1) - 1e-9:
            k += 1
        res[slots[k]].append(o)
        acc += cost(o)
    return res


# ---------------------------------------------------------------- one pipelined step
def step(r, checked=True):
    """Step s with s % 8 == r: every buffer index and LDS offset is static for a given r.
    Unchecked (the fast body), the two block sums go into L without the range check."""
    p, q = r & 1, (r & 1) ^ 1
    x1 = r + 1            # V block read in H1 (block s + 1: same parity and tile position)
    x3 = r + 3            # K block read in H2 (block s + 3)
    barrier = (r % 4) == 3
    out = [f"; ---- step r={r} (s = 8j + {r})"]
    loads = []
    if barrier:
        nb = ((x1 // 4) + 1) & 1           # buffers of the next V and K tiles
        out.append("s_waitcnt vmcnt(0) lgkmcnt(0)")
        out.append("s_barrier")
        loads = (tile_load_pairs(VDESC, VBUF + nb * TILE_BYTES, range(8)) +
                 tile_load_pairs(KDESC, KBUF + nb * TILE_BYTES, range(8)))
    else:
        out.append("s_waitcnt lgkmcnt(0)")
    li = 0
    # ---------------- H1: S(s+1,1) [KF[q]] and S(s+2,0) [KF[p]]
    mf = []
    for u in range(8):
        mf.append(mfma_s(q, 1, u))
        mf.append(mfma_s(p, 0, u))
    reads = vreads(x1)
    plan = place(merge(softmax_part(q, 0, 4, 8), softmax_part(p, 1, 4, 8)), list(range(16)))
    for k in range(16):
        if li < len(loads) and k % 2 == 1:
            out.append(loads[li][0])
        out.append(mf[k])
        if k == 8:
            out.append("s_waitcnt lgkmcnt(7)")
        out.append(reads[k])
        out.extend(plan.get(k, []))
        if li < len(loads) and k % 2 == 1:
            out.append(loads[li][1])
            li += 1
    # the range checks of the two blocks whose softmax ends here, with one branch
    if checked:
        out.extend(check_pair_and_fix(((q, 0), (p, 1)), f".Lf{r}"))
    else:
        out.extend(add_block_sums((q, 0), (p, 1)))
    # ---------------- H2: PV(s,1) [VF[p], P[p][1]] and PV(s+1,0) [VF[q], P[q][0]]
    kr = [kread(x3, u) for u in range(8)]
    # the ragged last block: the checked body masks its keys past the end (s = -inf); the fast
    # body leaves them at s = 0 (their K rows read as zero, their V rows too) and the kernel
    # takes their p out of the row sum afterwards
    masks = (mask_call(q, 1, MASK1, f".Lm{r}a") + mask_call(p, 0, MASK0, f".Lm{r}b")
             if checked else [])
    valu = masks + merge(softmax_part(q, 1, 0, 4), softmax_part(p, 0, 0, 4))
    # slots 1-14: the half's last MFMA slot, which the loop control and the next step's LDS
    # wait follow, carries no softmax work (0.7% faster than slots 1-15, measured on MI355X)
    plan = place(valu, list(range(1, 15)))
    out.append("s_waitcnt lgkmcnt(7)")       # V(s+1) reads 0..8 landed (h2 = 0 fragments)
    mf = []
    for h2 in range(2):
        for e in range(4):
            mf.append(mfma_pv(p, 1, e, h2))
            mf.append(mfma_pv(q, 0, e, h2))
    for k in range(16):
        if k == 9:
            out.append("s_waitcnt lgkmcnt(8)")   # all V(s+1) reads landed (h2 = 1 fragments)
        if li < len(loads) and k % 2 == 1:
            out.append(loads[li][0])
        out.append(mf[k])
        if 1 <= k <= 8:
            out.append(kr[k - 1])
        out.extend(plan.get(k, []))
        if li < len(loads) and k % 2 == 1:
            out.append(loads[li][1])
            li += 1
    assert li == len(loads)
    if barrier:
        out.extend(desc_advance(VDESC) + desc_advance(KDESC))
    out.append(f"s_cmp_eq_u32 {s(STEP)}, {s(LAST)}")
    out.append(f"s_cbranch_scc1 .Lexit{q}")
    out.append(f"s_add_u32 {s(STEP)}, {s(STEP)}, 1")
    return out


# ---------------------------------------------------------------- subroutines
def fix_routine(par, qb):
    """Rare path (vcc = lanes whose block sum is out of range): the two lanes of a query take
    the block's true max as the new reference if either needs it, rescale O and L by
    2^(m_old - m_new), and recompute the block."""
    out = [f".Lfix{par}{qb}:", "s_nop 7", "s_nop 7"]
    sb = S(par, qb)
    t0, t1, t2, t3, t4 = T0, T0 + 1, T0 + 2, T0 + 3, T0 + 4
    out.append(f"v_cndmask_b32_e64 {v(t0)}, 0, 1, vcc")
    out.append(f"v_max3_f32 {v(t1)}, {v(sb)}, {s(NINF)}, {v(sb + 1)}")
    for j in range(2, 16, 2):
        out.append(f"v_max3_f32 {v(t1)}, {v(t1)}, {v(sb + j)}, {v(sb + j + 1)}")
    out.append("s_waitcnt lgkmcnt(0)")
    out.append(f"ds_bpermute_b32 {v(t2)}, {v(VAX)}, {v(t0)}")
    out.append(f"ds_bpermute_b32 {v(t3)}, {v(VAX)}, {v(t1)}")
    out.append("s_waitcnt lgkmcnt(0)")
    out.append(f"v_cmp_ne_u32_e64 {s(STMP, 2)}, 0, {v(t2)}")
    out.append(f"s_or_b64 vcc, vcc, {s(STMP, 2)}")
    out.append(f"v_max_f32 {v(t3)}, {v(t3)}, {v(t3)}")
    out.append(f"v_max_f32 {v(t3)}, {v(t1)}, {v(t3)}")
    out.append(f"v_mul_f32 {v(t3)}, {s(SC)}, {v(t3)}")
    out.append(f"v_max_f32 {v(t4)}, {v(M + qb)}, {v(M + qb)}")
    out.append(f"v_max_f32 {v(t3)}, {v(t4)}, {v(t3)}")
    out.append(f"v_cndmask_b32 {v(t4)}, {v(M + qb)}, {v(t3)}, vcc")     # m_new
    out.append(f"v_sub_f32 {v(t3)}, {v(M + qb)}, {v(t4)}")
    out.append(f"v_exp_f32 {v(t3)}, {v(t3)}")
    out.append("s_nop 0")
    out.append(f"v_cndmask_b32 {v(t3)}, 1.0, {v(t3)}, vcc")              # alpha
    out.append(f"v_mul_f32 {v(L + qb)}, {v(L + qb)}, {v(t3)}")
    tmp = [TMP(0) + i for i in range(8)]
    regs = [O(qb, e) + j for e in range(4) for j in range(16)]
    for k in range(0, 64, 8):
        for i in range(8):
            out.append(f"v_accvgpr_read_b32 {v(tmp[i])}, {a(regs[k + i])}")
        for i in range(8):
            out.append(f"v_mul_f32 {v(tmp[i])}, {v(tmp[i])}, {v(t3)}")
        for i in range(8):
            out.append(f"v_accvgpr_write_b32 {a(regs[k + i])}, {v(tmp[i])}")
    out.append(f"v_mov_b32 {v(M + qb)}, {v(t4)}")
    out.append(f"v_xor_b32 {v(NEGM + qb)}, 0x80000000, {v(t4)}")
    out.extend(softmax_full(par, qb))
    out.append("s_nop 1")
    out.append(f"s_setpc_b64 {s(RET, 2)}")
    return out


def mask_routine(par, qb):
    """Keys at or past n_tokens in the ragged last block get s = -inf (their p is exactly 0)."""
    out = [f".Lmask{par}{qb}:", "s_nop 7", "s_nop 7"]
    sb = S(par, qb)
    for j in range(16):
        cj = 16 * (j >> 3) + 8 * ((j >> 2) & 1) + (j & 3)
        out.append(f"v_cmp_le_i32 vcc, {-cj}, {v(VT)}")
        out.append(f"v_cndmask_b32 {v(sb + j)}, {v(sb + j)}, {v(VNINF)}, vcc")
    out.append(f"s_setpc_b64 {s(RET, 2)}")
    return out


# ---------------------------------------------------------------- prologue / epilogue
def prologue(checked=True):
    """Loads V tiles 0, 1 and K tiles -1 (blocks 0, 1 only) and 0; computes S(0, *) and
    S(1, 0), the whole softmax of (0, 0), PV(0, 0), pairs 0..3 of softmax(0, 1) and (1, 0);
    reads K(2) and V(0); then refills K buffer 1 with K tile 1.  Leaves the state step 0
    expects.  Unchecked, the reference max of both query blocks is first set from key
    block 0."""
    out = ["; ---- prologue",
           f"s_mov_b32 {s(M0SAVE)}, m0",
           f"s_mov_b32 {s(NINF)}, 0xff800000",
           f"v_mov_b32 {v(VNINF)}, 0xff800000",
           f"s_mov_b32 {s(STEP)}, 0",
           f"s_sub_u32 {s(MASK0)}, {s(MASK1)}, 1",
           f"s_getpc_b64 {s(RET, 2)}",
           ".Lanchor:"]
    for par in range(2):
        for qb in range(2):
            k = par * 2 + qb
            out += [f"s_add_u32 {s(FIXA + 2 * k)}, {s(RET)}, .Lfix{par}{qb}-.Lanchor",
                    f"s_addc_u32 {s(FIXA + 2 * k + 1)}, {s(RET + 1)}, 0",
                    f"s_add_u32 {s(MASKA + 2 * k)}, {s(RET)}, .Lmask{par}{qb}-.Lanchor",
                    f"s_addc_u32 {s(MASKA + 2 * k + 1)}, {s(RET + 1)}, 0"]
    def emit(pairs):
        for m0, ld in pairs:
            out.extend([m0, "s_nop 0", ld])
    emit(tile_load_pairs(VDESC, VBUF, range(8)))                     # V tile 0 -> buffer 0
    emit(tile_load_pairs(KDESC, KBUF + TILE_BYTES, range(4, 8)))     # K tile -1: blocks 0, 1
    out.extend(desc_advance(KDESC))
    emit(tile_load_pairs(KDESC, KBUF, range(8)))                     # K tile 0 -> buffer 0
    out.extend(desc_advance(KDESC) + desc_advance(VDESC))
    emit(tile_load_pairs(VDESC, VBUF + TILE_BYTES, range(8)))        # V tile 1 -> buffer 1
    out.extend(desc_advance(VDESC))
    out += ["s_waitcnt vmcnt(0)", "s_barrier"]
    for u in range(8):
        out.append(kread(0, u))
    out.append("s_waitcnt lgkmcnt(0)")
    for u in range(8):
        out.append(kread(1, u))
    for u in range(8):                                               # S(0, 0)
        out.append(mfma_s(0, 0, u))
    out.append("s_waitcnt lgkmcnt(0)")
    vr = vreads(0)
    for u in range(8):                                               # S(0, 1), S(1, 0)
        out.append(mfma_s(0, 1, u))
        out.append(mfma_s(1, 0, u))
        if u == 4:
            out.append("s_waitcnt lgkmcnt(7)")
        out.extend(vr[2 * u:2 * u + 2])
    out += ["s_nop 7"]
    if not checked:
        out += ["s_nop 7", "s_nop 7"]           # the S(0, 1) MFMAs just issued -> VALU reads
        out += init_reference_max(0, 0) + init_reference_max(0, 1)
    out.extend(softmax_full(0, 0))
    out.extend(check_and_fix(0, 0, ".Lfp0") if checked else add_block_sums((0, 0)))
    out.append("s_waitcnt lgkmcnt(0)")
    out.append("s_nop 1")
    for h2 in range(2):
        for e in range(4):
            out.append(mfma_pv(0, 0, e, h2))                         # PV(0, 0)
    for u in range(8):
        out.append(kread(2, u))                                      # K(2) -> KF[0]
    out.append("s_nop 7")
    out.extend(merge(softmax_part(0, 1, 0, 4), softmax_part(1, 0, 0, 4)))
    out += ["s_waitcnt lgkmcnt(0)", "s_barrier"]                     # K tile -1 no longer read
    emit(tile_load_pairs(KDESC, KBUF + TILE_BYTES, range(8)))        # K tile 1 -> buffer 1
    out.extend(desc_advance(KDESC))
    return out


def epilogue(checked=True):
    """After the last step (s = n_blocks - 2): pairs 4..7 of softmax(s+1, 1), then PV(s+1, 1)."""
    out = []
    for x in range(2):
        out.append(f".Lexit{x}:")
        out.append("s_waitcnt lgkmcnt(0)")
        out.extend(softmax_part(x, 1, 4, 8))
        out.extend(check_and_fix(x, 1, f".Lfe{x}") if checked else add_block_sums((x, 1)))
        out.append("s_nop 1")
        for h2 in range(2):
            for e in range(4):
                out.append(mfma_pv(x, 1, e, h2))
        out.append("s_branch .Ldone")
    return out


def generate(checked=True):
    """The whole asm body, one instruction or label per list entry.  checked=False gives the
    fast body: no range check inside the loop, every label renamed (.LF...) so that both
    bodies can sit in one kernel."""
    body = []
    body.extend(prologue(checked))
    body.append(".Lloop:")
    for r in range(8):
        body.extend(step(r, checked))
    body.append("s_branch .Lloop")
    body.extend(epilogue(checked))
    for par in range(2):
        for qb in range(2):
            body.extend(fix_routine(par, qb))
            body.extend(mask_routine(par, qb))
    body.extend(call_stubs(body))
    body += [".Ldone:",
             "s_waitcnt vmcnt(0) lgkmcnt(0)",
             f"s_mov_b32 m0, {s(M0SAVE)}",
             "s_nop 15",                        # MFMA results -> the compiler's reads of O
             "s_nop 7"]
    if not checked:
        body = [re.sub(r"\.L(\w+)", r".LF\1", l) for l in body]
    return body


def clobbered():
    """Registers the body writes besides its in/out operands: {'v': set, 'a': set, 's': set}."""
    return {"v": set(range(0, 160)) | (set(range(192, NV_END)) - {195}),
            "a": set(range(192, 256)),
            "s": {STEP, M0SAVE, MASK0, MASK0 + 1} | set(range(NINF, 76))}


def clobber_list():
    c = clobbered()
    out = [f'"v{i}"' for i in sorted(c["v"])] + [f'"a{i}"' for i in sorted(c["a"])]
    out += [f'"s{i}"' for i in sorted(c["s"])]
    out += ['"vcc"', '"scc"', '"memory"']
    return ", ".join(out)


def write(path):
    with open(path, "w") as f:
        f.write("// Generated by attn_loop_gen.py: the key loop of attn_pipe.hip (inline asm bodies).\n")
        for name, checked in (("HSA_ATTN_LOOP_ASM", True), ("HSA_ATTN_LOOP_FAST_ASM", False)):
            f.write(f"#define {name} \\\n")
            for l in generate(checked):
                l2 = l.replace("\\", "\\\\").replace('"', '\\"')
                f.write(f'  "{l2}\\n" \\\n')
            f.write("  \"\"\n")
        f.write(f"#define HSA_ATTN_LOOP_CLOBBERS {clobber_list()}\n")


if __name__ == "__main__":
    if len(sys.argv) > 1:
        write(sys.argv[1])
    else:
        print("\n".join(generate()))
