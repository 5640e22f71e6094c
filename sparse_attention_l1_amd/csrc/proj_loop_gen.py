"""Generates the reduction loop of the fused QKV projection (proj.hip) as gfx950 assembly.

The projection of the active rows ("Technische Samenvatting: Heterogene Staptoewijzing (HSA)
voor Efficiënte Videogeneratie", §2.2 items 1-2) is a plain GEMM, Y = X_A W^T, with both
operands K-contiguous.  A workgroup of 4 wavefronts (one per SIMD) owns a 256 x 256 tile of Y;
wavefront (wm, wn) owns the 128 x 128 quarter at rows 128 wm, columns 128 wn, as 8 x 8 blocks
of v_mfma_f32_16x16x32_bf16 whose fp32 accumulators fill all 256 AGPRs.  The 16x16x32 form
does the same work per cycle as 32x32x16 but draws less power per flop, so the chip holds a
higher clock under it (measured on MI355X: 2.07 against 1.86 GHz for a loop of MFMAs alone).

The MFMAs take the W fragment as their A operand and the X fragment as their B operand, so
each block holds Y^T: a lane owns one row of Y and four consecutive columns per block, which
the epilogue writes as one 8-byte unit.

The reduction dimension walks in stages of 64 elements (2 k-steps of 32):

  k-step 0 of a stage: its 64 MFMAs (fragment slot 0) interleaved with the 16 LDS reads of
                       k-step 1's fragments (slot 1) and, per SPLIT, the rest of the refill of
                       the other buffer that the previous stage began;
  k-step 1:            first a wait for this wavefront's tile loads and LDS reads and a barrier
                       (after it every wavefront has finished reading this stage's buffer and
                       the next stage's tile has landed), then its 64 MFMAs interleaved with
                       the reads of the next stage's k-step 0 and the first tile loads of the
                       stage after next, into the buffer just freed, one every LOAD_EVERY
                       MFMAs so that the four wavefronts' L2 requests arrive at an even rate.

Rotated start.  A tile begins its reduction at stage rot (chosen per tile by the kernel) and
wraps around to stage 0 after the last one, so that the tiles running at the same time read
different 128-byte columns of X and W.  When the row pitch is a multiple of 256 bytes (model
dim 5120, say) and every tile walks from stage 0, the lines all compute units fetch at once
fall on a few memory channels; spreading the starts over 64 positions made such shapes 14%
faster on MI355X (and shapes with other pitches no slower).  The sum over stages is the same
set of partial products in a rotated order.

Stages are double buffered in LDS (64 KB each: 256 rows x 128 bytes of X, the same of W).
Tiles travel global -> LDS through buffer loads with an LDS destination; the descriptors cover
exactly the tile's valid rows, so rows past the end of X or W read as zero, and a stage past
the end of the reduction gets an empty range.  Rows are 128 bytes with the 16-byte chunk
c stored at slot c ^ ((row >> 1) & 7), which keeps each phase of a fragment read on distinct
LDS banks.  A fragment read of row block i is one address register per k-step plus the
immediate offset 2048 i (16 rows of 128 bytes).  The loop body is unrolled over two stages so
that every LDS offset is an immediate.

Register map (per lane):  VGPR  fragments 0-127 (slot, X row blocks, W column blocks), LDS read
addresses 128-131, tile-load offsets 132-139;  AGPR  accumulators 0-255;  SGPR 40-55
(descriptors, m0 base, stage counter, wrap point).
"""
import sys

# ---------------------------------------------------------------- register map
def XF(slot, i):           # X fragment of row block i (B operand): 4 VGPRs
    return slot * 64 + i * 4
def WF(slot, j):           # W fragment of column block j (A operand): 4 VGPRs
    return slot * 64 + 32 + j * 4
XADDR = 128                # 2: [u] LDS byte address of the lane's X fragment, k-step u, block 0
WADDR = 130                # 2: the same for W (includes the W region base)
XVOFF = 132                # 8: buffer offset of tile-load instruction i (X and W alike: both
WVOFF = XVOFF              #    tiles have rows of model-dim elements)
def ACC(i, j):             # accumulator of block (i, j): 4 AGPRs
    return (i * 8 + j) * 4

XDESC = 40                 # s[40:43] buffer descriptor of the X tile (advances per stage)
WDESC = 44                 # s[44:47] same for W
M0BASE = 48                # LDS byte address of this wavefront's first tile-load slot
STAGE = 49                 # stage counter
NSTAGE = 50                # number of stages (model dim / 64)
M0SAVE = 51
KADV = 52                  # descriptor advance per stage (128 bytes)
TMPS = 53
WRAPT = 54                 # the stage at which the descriptors wrap (nstage - rot)
WRAPB = 55                 # bytes they move back then (nstage * 128)

XBUF = (0, 32768)          # LDS byte offset of the X half of stage buffer 0 / 1
WBUF = (65536, 98304)      # the W halves
LOAD_BYTES = 4096          # one tile-load instruction of the 4 wavefronts: 32 rows x 128 B
BLOCK_BYTES = 2048         # 16 rows of 128 bytes: the offset between fragment row blocks
KSTEPS = 2                 # k-steps of 32 per 64-element stage
READS = 16                 # fragment reads per k-step


def v(r, n=1):
    return f"v{r}" if n == 1 else f"v[{r}:{r + n - 1}]"
def a(r, n=1):
    return f"a{r}" if n == 1 else f"a[{r}:{r + n - 1}]"
def s(r, n=1):
    return f"s{r}" if n == 1 else f"s[{r}:{r + n - 1}]"


# ---------------------------------------------------------------- instruction groups
def mfma(slot, i, j):
    return (f"v_mfma_f32_16x16x32_bf16 {a(ACC(i, j), 4)}, {v(WF(slot, j), 4)}, "
            f"{v(XF(slot, i), 4)}, {a(ACC(i, j), 4)}")


def reads(buf, u, slot):
    """The 16 fragment reads of k-step u of the stage in buffer buf, into slot: X row blocks
    and W column blocks alternately, in the order the MFMAs of that k-step use them."""
    out = []
    for b in range(8):
        out.append(f"ds_read_b128 {v(XF(slot, b), 4)}, {v(XADDR + u)} "
                   f"offset:{XBUF[buf] + b * BLOCK_BYTES}")
        out.append(f"ds_read_b128 {v(WF(slot, b), 4)}, {v(WADDR + u)} "
                   f"offset:{WBUF[buf] - WBUF[0] + b * BLOCK_BYTES}")
    return out


def loads(buf):
    """(m0 write, load) pairs filling stage buffer buf: 8 X and 8 W instructions per wavefront."""
    out = []
    for i in range(8):
        out.append((f"s_add_u32 m0, {s(M0BASE)}, {XBUF[buf] + i * LOAD_BYTES}",
                    f"buffer_load_dwordx4 {v(XVOFF + i)}, {s(XDESC, 4)}, 0 offen lds"))
        out.append((f"s_add_u32 m0, {s(M0BASE)}, {WBUF[buf] + i * LOAD_BYTES}",
                    f"buffer_load_dwordx4 {v(WVOFF + i)}, {s(WDESC, 4)}, 0 offen lds"))
    return out


def advance(ahead):
    """Both descriptors move one stage (128 bytes along the reduction) and wrap back to the
    start of the rows when the stage the next load fetches (STAGE + ahead) is WRAPT, the first
    one past the end of the rows for a tile that began at stage rot = nstage - WRAPT; once
    that stage is past the last one, their ranges become empty."""
    out = []
    for d in (XDESC, WDESC):
        out += [f"s_add_u32 {s(d)}, {s(d)}, {s(KADV)}",
                f"s_addc_u32 {s(d + 1)}, {s(d + 1)}, 0"]
    out += [f"s_add_u32 {s(TMPS)}, {s(STAGE)}, {ahead}",
            f"s_cmp_eq_u32 {s(TMPS)}, {s(WRAPT)}",
            f"s_cselect_b32 {s(TMPS)}, {s(WRAPB)}, 0"]
    for d in (XDESC, WDESC):
        out += [f"s_sub_u32 {s(d)}, {s(d)}, {s(TMPS)}",
                f"s_subb_u32 {s(d + 1)}, {s(d + 1)}, 0"]
    out += [f"s_add_u32 {s(TMPS)}, {s(STAGE)}, {ahead}",
            f"s_cmp_ge_u32 {s(TMPS)}, {s(NSTAGE)}",
            f"s_cselect_b32 {s(XDESC + 2)}, 0, {s(XDESC + 2)}",
            f"s_cselect_b32 {s(WDESC + 2)}, 0, {s(WDESC + 2)}"]
    return out


SPLIT = 16                 # tile loads of a refill issued in k-step 1 after the barrier; the
                           # rest go into the next stage's k-step 0
LOAD_EVERY = 4             # MFMAs between two tile loads
READ_EVERY = 2             # MFMAs between two fragment reads


def _kstep(mf, rd, ld):
    """Interleaves one k-step: a read after every READ_EVERY-th MFMA and a tile load (its m0
    write one MFMA ahead) after every LOAD_EVERY-th, starting at the second MFMA."""
    out = []
    for k, m in enumerate(mf):
        li = (k - 1) // LOAD_EVERY if (k - 1) % LOAD_EVERY == 0 and k >= 1 else None
        if li is not None and li < len(ld):
            out.append(ld[li][0])
        out.append(m)
        if k % READ_EVERY == 0 and k // READ_EVERY < len(rd):
            if k // READ_EVERY == 15:
                out.append("s_waitcnt lgkmcnt(14)")   # at most 15 LDS reads in flight
            out.append(rd[k // READ_EVERY])
        if li is not None and li < len(ld):
            out.append(ld[li][1])
    return out


def stage(par):
    """One stage in buffer par: k-step 0 finishes the refill of the other buffer that the
    previous stage began (if SPLIT < 16); k-step 1 begins the refill of this one."""
    mf = lambda u: [mfma(u, i, j) for i in range(8) for j in range(8)]
    out = [f"; ---- stage in buffer {par}", "s_waitcnt lgkmcnt(0)"]
    out += _kstep(mf(0), reads(par, 1, 1), loads(par ^ 1)[SPLIT:])
    if SPLIT < 16:
        out += advance(2)                 # the refill of stage STAGE + 1 is complete
    out += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"]
    out += _kstep(mf(1), reads(par ^ 1, 0, 0), loads(par)[:SPLIT])
    if SPLIT == 16:
        out += advance(3)                 # the refill of stage STAGE + 2 is complete
    return out


def prologue():
    """Stage 0 into buffer 0 and the first part of stage 1 into buffer 1 (what the k-step 1 of
    a stage -1 would have loaded; the first stage's k-step 0 loads the rest, as in steady
    state)."""
    out = ["; ---- prologue",
           # the previous tile's stores are on the same counter as the tile loads: wait for
           # them here, so that the counts below are this tile's loads only
           "s_waitcnt vmcnt(0)",
           f"s_mov_b32 {s(M0SAVE)}, m0",
           f"s_mov_b32 {s(KADV)}, 128",
           f"s_mov_b32 {s(STAGE)}, 0"]
    for m0, ld in loads(0):
        out += [m0, "s_nop 0", ld]
    out += advance(1)
    for m0, ld in loads(1)[:SPLIT]:
        out += [m0, "s_nop 0", ld]
    if SPLIT == 16:
        out += advance(2)
    out += [f"s_waitcnt vmcnt({SPLIT})", "s_barrier"]   # stage 0 landed for every wavefront
    rd = reads(0, 0, 0)
    out += rd[:15] + ["s_waitcnt lgkmcnt(14)"] + rd[15:]
    return out


def generate():
    body = prologue() + [".Lploop:"]
    for par in range(2):
        body += stage(par)
        body += [f"s_add_u32 {s(STAGE)}, {s(STAGE)}, 1",
                 f"s_cmp_eq_u32 {s(STAGE)}, {s(NSTAGE)}",
                 "s_cbranch_scc1 .Lpdone"]
    body += ["s_branch .Lploop",
             ".Lpdone:",
             "s_waitcnt vmcnt(0) lgkmcnt(0)",
             f"s_mov_b32 m0, {s(M0SAVE)}",
             "s_nop 15",                        # MFMA results -> the compiler's reads of Y
             "s_nop 7"]
    return body


def clobbered():
    """Registers the body writes besides its in/out operands: {'v': set, 'a': set, 's': set}."""
    return {"v": set(range(0, 128)), "a": set(), "s": {STAGE, M0SAVE, KADV, TMPS}}


def clobber_list():
    c = clobbered()
    out = [f'"v{i}"' for i in sorted(c["v"])] + [f'"s{i}"' for i in sorted(c["s"])]
    out += ['"vcc"', '"scc"', '"memory"']
    return ", ".join(out)


def write(path):
    body = generate()
    with open(path, "w") as f:
        f.write("// Generated by proj_loop_gen.py: the reduction loop of proj.hip (inline asm body).\n")
        f.write("#define HSA_PROJ_LOOP_ASM \\\n")
        for l in body:
            l2 = l.replace("\\", "\\\\").replace('"', '\\"')
            f.write(f'  "{l2}\\n" \\\n')
        f.write("  \"\"\n")
        f.write(f"#define HSA_PROJ_LOOP_CLOBBERS {clobber_list()}\n")


if __name__ == "__main__":
    if len(sys.argv) > 1:
        write(sys.argv[1])
    else:
        print("\n".join(generate()))
