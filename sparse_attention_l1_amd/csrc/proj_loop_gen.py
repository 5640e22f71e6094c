"""Generates the reduction loop of the fused QKV projection (proj.hip) as gfx950 assembly.

The projection of the active rows ("Technische Samenvatting: Heterogene Staptoewijzing (HSA)
voor Efficiënte Videogeneratie", §2.2 items 1-2) is a plain GEMM, Y = X_A W^T, with both
operands K-contiguous.  A workgroup of 4 wavefronts (one per SIMD) owns a 256 x 256 tile of Y;
wavefront (wm, wn) owns the 128 x 128 quarter at rows 128 wm, columns 128 wn, as 4 x 4 blocks
of v_mfma_f32_32x32x16_bf16 whose fp32 accumulators fill all 256 AGPRs.

The MFMAs take the W fragment as their A operand and the X fragment as their B operand, so
each block holds Y^T: a lane owns one row of Y and, per group of four registers, four
consecutive columns, which the epilogue stores as one 8-byte write.

The reduction dimension walks in stages of 64 elements (4 k-steps of 16):

  k-step u of a stage: the 16 MFMAs of fragment slot u & 1, each followed by one of the 8 LDS
                       reads of the next k-step's fragments (slot (u + 1) & 1);
  k-step 3:            first a wait for this wavefront's tile loads and LDS reads and a barrier
                       (after it every wavefront has finished reading this stage's buffer and
                       the next stage's tile has landed), then its MFMAs interleaved with the
                       reads of the next stage's k-step 0 and the first 6 of the 16 tile loads
                       of the stage after next, into the buffer just freed;
  k-steps 0 and 1:     the other 5 + 5 of those tile loads, one per MFMA.

Spreading the tile loads over three k-steps instead of one keeps the L2 requests of the
workgroup's four wavefronts at an even rate (5-8% faster than issuing all 16 at once); the
last ones still have a full k-step to land before the next barrier.

Stages are double buffered in LDS (64 KB each: 256 rows x 128 bytes of X, the same of W).
Tiles travel global -> LDS through buffer loads with an LDS destination; the descriptors cover
exactly the tile's valid rows, so rows past the end of X or W read as zero, and a stage past
the end of the reduction gets an empty range.  Rows are 128 bytes with the 16-byte chunk
c stored at slot c ^ ((row >> 1) & 7), which keeps each 16-lane phase of a fragment read on
distinct LDS banks.  The loop body is unrolled over two stages so that every LDS offset is an
immediate.

Register map (per lane):  VGPR  fragments 0-63 (slot, A rows / B rows), LDS read addresses
64-95, tile-load offsets 96-111;  AGPR  accumulators 0-255;  SGPR 40-53 (descriptors, m0 base,
stage counter).
"""
import sys

# ---------------------------------------------------------------- register map
def XF(slot, i):           # X fragment of row block i (B operand): 4 VGPRs
    return slot * 32 + i * 4
def WF(slot, j):           # W fragment of column block j (A operand): 4 VGPRs
    return slot * 32 + 16 + j * 4
XADDR = 64                 # 16: [i*4 + u] LDS byte address of X fragment (i, k-step u), buffer 0
WADDR = 80                 # 16: [j*4 + u] the same for W (includes the W region base)
XVOFF = 96                 # 8: buffer offset of X tile-load instruction i
WVOFF = 104                # 8: the same for W
def ACC(i, j):             # accumulator of block (i, j): 16 AGPRs
    return (i * 4 + j) * 16

XDESC = 40                 # s[40:43] buffer descriptor of the X tile (advances per stage)
WDESC = 44                 # s[44:47] same for W
M0BASE = 48                # LDS byte address of this wavefront's first tile-load slot
STAGE = 49                 # stage counter
NSTAGE = 50                # number of stages (model dim / 64)
M0SAVE = 51
KADV = 52                  # descriptor advance per stage (128 bytes)
TMPS = 53

XBUF = (0, 32768)          # LDS byte offset of the X half of stage buffer 0 / 1
WBUF = (65536, 98304)      # the W halves
LOAD_BYTES = 4096          # one tile-load instruction of the 4 wavefronts: 32 rows x 128 B


def v(r, n=1):
    return f"v{r}" if n == 1 else f"v[{r}:{r + n - 1}]"
def a(r, n=1):
    return f"a{r}" if n == 1 else f"a[{r}:{r + n - 1}]"
def s(r, n=1):
    return f"s{r}" if n == 1 else f"s[{r}:{r + n - 1}]"


# ---------------------------------------------------------------- instruction groups
def mfma(slot, i, j):
    return (f"v_mfma_f32_32x32x16_bf16 {a(ACC(i, j), 16)}, {v(WF(slot, j), 4)}, "
            f"{v(XF(slot, i), 4)}, {a(ACC(i, j), 16)}")


def reads(buf, u, slot):
    """The 8 fragment reads of k-step u of the stage in buffer buf, into slot."""
    out = [f"ds_read_b128 {v(XF(slot, i), 4)}, {v(XADDR + i * 4 + u)} offset:{XBUF[buf]}"
           for i in range(4)]
    out += [f"ds_read_b128 {v(WF(slot, j), 4)}, {v(WADDR + j * 4 + u)} offset:{WBUF[buf] - WBUF[0]}"
            for j in range(4)]
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
    """Both descriptors move one stage (128 bytes along the reduction); once the stage the next
    load would fetch (STAGE + ahead) is past the end, their ranges become empty."""
    out = []
    for d in (XDESC, WDESC):
        out += [f"s_add_u32 {s(d)}, {s(d)}, {s(KADV)}",
                f"s_addc_u32 {s(d + 1)}, {s(d + 1)}, 0"]
    out += [f"s_add_u32 {s(TMPS)}, {s(STAGE)}, {ahead}",
            f"s_cmp_ge_u32 {s(TMPS)}, {s(NSTAGE)}",
            f"s_cselect_b32 {s(XDESC + 2)}, 0, {s(XDESC + 2)}",
            f"s_cselect_b32 {s(WDESC + 2)}, 0, {s(WDESC + 2)}"]
    return out


SPLIT = (0, 6, 11, 16)     # tile loads of a refill: [0, 6) after the barrier, [6, 11) and [11, 16)
                           # in the next stage's k-steps 0 and 1


def stage(par):
    """One stage in buffer par: 4 k-steps of 16 MFMAs; k-steps 0 and 1 finish the refill of
    the other buffer that the previous stage began, k-step 3 begins the refill of this one."""
    out = [f"; ---- stage in buffer {par}"]
    for u in range(4):
        if u < 3:
            out.append("s_waitcnt lgkmcnt(0)")
            rd = reads(par, u + 1, (u + 1) & 1)
            ld = loads(par ^ 1)[SPLIT[u + 1]:SPLIT[u + 2]] if u + 2 < len(SPLIT) else []
        else:
            out += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"]
            rd, ld = reads(par ^ 1, 0, 0), loads(par)[SPLIT[0]:SPLIT[1]]
        mf = [mfma(u & 1, i, j) for i in range(4) for j in range(4)]
        for k in range(16):
            if k < len(ld):
                out.append(ld[k][0])          # m0 write, one instruction ahead of its load
            out.append(mf[k])
            if k < len(rd):
                out.append(rd[k])
            if k < len(ld):
                out.append(ld[k][1])
        if u == len(SPLIT) - 3:
            out += advance(2)                 # the refill of stage STAGE + 1 is complete
    return out


def prologue():
    """Stage 0 into buffer 0 and the first part of stage 1 into buffer 1 (the first stage's
    k-steps 0 and 1 load the rest, as in steady state)."""
    out = ["; ---- prologue",
           f"s_mov_b32 {s(M0SAVE)}, m0",
           f"s_mov_b32 {s(KADV)}, 128",
           f"s_mov_b32 {s(STAGE)}, 0"]
    for m0, ld in loads(0):
        out += [m0, "s_nop 0", ld]
    out += advance(1)
    for m0, ld in loads(1)[SPLIT[0]:SPLIT[1]]:
        out += [m0, "s_nop 0", ld]
    out += [f"s_waitcnt vmcnt({SPLIT[1]})", "s_barrier"]   # stage 0 landed for every wavefront
    out += reads(0, 0, 0)
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
    return {"v": set(range(0, 64)), "a": set(), "s": {STAGE, M0SAVE, KADV, TMPS}}


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
