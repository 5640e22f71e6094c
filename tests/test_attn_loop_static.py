"""The generated key loop of the head_dim 128 attention kernel, checked without a GPU.

The loop is hand-scheduled assembly (attn_loop_gen.py), so the wait states the hardware needs
between dependent instructions, the LDS counter waits, the registers it may touch and its LDS
offsets are checked here statically; a planted mistake of each kind must be caught.
"""
import os

import numpy as np
import pytest

import loop_checker as lc

GEN = lc.load_generator()
HIP = open(os.path.join(lc.CSRC, "attn_pipe.hip")).read()


@pytest.mark.parametrize("checked", [True, False], ids=["checked", "fast"])
def test_hazards_and_lds_counters(checked):
    assert lc.check_hazards(GEN, checked) == []


@pytest.mark.parametrize("checked", [True, False], ids=["checked", "fast"])
def test_registers_are_declared(checked):
    assert lc.check_registers(GEN, HIP, checked) == []


@pytest.mark.parametrize("checked", [True, False], ids=["checked", "fast"])
def test_lds_offsets_in_bounds(checked):
    assert lc.check_lds_bounds(GEN, checked) == []


def test_fast_body_shape():
    """The fast body: the same loop without any range check, ragged-block test or
    data-dependent branch (the same MFMAs, LDS reads, tile loads and barriers in the same
    order, and as many exponentials), its labels distinct from the checked body's, and each
    query block's reference max set from key block 0 before that block's first
    exponential."""
    fast, checked = GEN.generate(False), GEN.generate(True)
    assert not any(l.startswith(("s_cbranch_vccnz", "v_cmp_nge_f32")) for l in fast)
    assert any(l.startswith("s_cbranch_vccnz") for l in checked)
    labels = lambda body: {l[:-1] for l in body if l.endswith(":")}
    assert labels(fast) and not labels(fast) & labels(checked)
    loop_f = fast[fast.index(".LFloop:"):fast.index("s_branch .LFloop")]
    loop_c = checked[checked.index(".Lloop:"):checked.index("s_branch .Lloop")]
    strip = lambda body: [l for l in body if l.startswith(("v_mfma", "ds_read", "buffer_load", "s_barrier"))]
    assert strip(loop_f) == strip(loop_c)
    n_exp = lambda body: sum(l.startswith("v_exp") for l in body)
    assert n_exp(loop_f) == n_exp(loop_c)
    assert not any(l.startswith("s_cbranch_scc1") and "_call" in l for l in loop_f)
    assert any(l.startswith("s_cbranch_scc1") and "_call" in l for l in loop_c)
    first_exp = next(i for i, l in enumerate(fast) if l.startswith("v_exp_f32"))
    for qb in (0, 1):
        sets_m = [i for i, l in enumerate(fast) if l.startswith(f"v_mov_b32 v{GEN.M + qb},")]
        assert sets_m and sets_m[0] < first_exp


def test_loop_shape():
    body = GEN.generate()
    mf = [l for l in body if l.startswith("v_mfma")]
    # per step: 16 S^T MFMAs (two chains of 8) and 16 P.V MFMAs; 8 unrolled steps
    loop = body[body.index(".Lloop:"):body.index("s_branch .Lloop")]
    assert sum(l.startswith("v_mfma_f32_32x32x16_bf16") for l in loop) == 8 * 32
    assert sum(l.startswith("v_mfma") for l in loop) == 8 * 32
    # two blocks per step, 8 rounded pairs each, read back as two fp32 values
    assert sum(l.startswith("v_and_b32") for l in loop) == 8 * 2 * 8
    assert sum(l.startswith("v_lshlrev_b32") for l in loop) == 8 * 2 * 8
    assert sum(l == "s_barrier" for l in loop) == 2                  # one per 4 steps
    assert sum(l.startswith("buffer_load") for l in loop) == 2 * 16  # V and K tile per barrier
    assert sum(l.startswith("v_exp_f32") for l in loop) == 8 * 2 * 16
    assert len(mf) > 0


def _with_patch(name, fn):
    orig = getattr(GEN, name)
    setattr(GEN, name, fn(orig))
    try:
        return lc.check_hazards(GEN)
    finally:
        setattr(GEN, name, orig)


def test_checker_catches_a_missing_lds_wait():
    errs = _with_patch("step", lambda f: lambda *a: [l for l in f(*a) if "lgkmcnt(8)" not in l])
    assert any("LDS result is in flight" in e for e in errs)


def test_checker_catches_a_missing_wait_state():
    # an exponential's result read by the very next instruction
    def early(f):
        def g(*a):
            out = []
            for l in f(*a):
                out.append(l)
                if l.startswith("v_exp_f32"):
                    out.append(f"v_mov_b32 v218, {l.split()[1].rstrip(',')}")
            return out
        return g
    errs = _with_patch("softmax_part", early)
    assert any("needs 1" in e for e in errs)


def test_checker_catches_an_early_mfma_read():
    # VALU reading an S^T accumulator right after the MFMA chain that writes it
    def early(f):
        def g(*a):
            out = f(*a)
            hits = [k for k, l in enumerate(out) if l.startswith("v_mfma") and "v[0:15]" in l.split(",")[0]]
            if not hits:
                return out
            i = max(hits)
            return out[:i + 1] + ["v_add_f32 v196, v0, v1"] + out[i + 1:]
        return g
    errs = _with_patch("step", early)
    assert any("needs 12" in e for e in errs)


def test_checker_catches_an_undeclared_register():
    orig = GEN.clobbered
    GEN.clobbered = lambda: {k: (s - {100} if k == "v" else s) for k, s in orig().items()}
    try:
        assert any("('v', 100)" in e for e in lc.check_registers(GEN, HIP))
    finally:
        GEN.clobbered = orig


def _bf16_rne(x):
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)


def _run_valu(ops, reg, sgpr):
    """Executes the softmax's VALU instructions on one lane (register contents as uint32 bits):
    fp32 FMA/add, exp2, RNE bf16 packing, and the integer read-back of the packed halves."""
    f = lambda r: np.uint32(reg[r]).view(np.float32)
    put = lambda r, x: reg.__setitem__(r, int(np.float32(x).view(np.uint32)))
    num = lambda t: int(t[1:]) if t.startswith("v") else None
    for op in ops:
        name, rest = op.split(None, 1)
        a = [t.strip() for t in rest.split(",")]
        if name == "v_fma_f32":
            sc = np.uint32(sgpr[int(a[2][1:])]).view(np.float32)
            put(num(a[0]), np.float32(np.float64(f(num(a[1]))) * np.float64(sc) + np.float64(f(num(a[3])))))
        elif name == "v_exp_f32":
            put(num(a[0]), np.exp2(f(num(a[1]))))
        elif name == "v_cvt_pk_bf16_f32":
            lo, hi = _bf16_rne(f(num(a[1]))), _bf16_rne(f(num(a[2])))
            reg[num(a[0])] = int(lo) | (int(hi) << 16)
        elif name == "v_and_b32":
            reg[num(a[0])] = int(a[1], 16) & reg[num(a[2])]
        elif name == "v_lshlrev_b32":
            reg[num(a[0])] = (reg[num(a[2])] << int(a[1])) & 0xFFFFFFFF
        elif name == "v_add_f32":
            put(num(a[0]), f(num(a[1])) + f(num(a[2])))
        else:
            raise AssertionError(op)


def test_block_sum_is_the_sum_of_the_rounded_p():
    """The generated softmax of a block leaves in LS the fp32 tree sum of exactly the bf16
    values written into its P registers (the weights the P.V MFMAs apply), and P holds
    bf16(2^(s*c - m)) for the block's 16 scores of this lane."""
    rng = np.random.default_rng(5)
    for par, qb in ((0, 0), (1, 1), (0, 1)):
        reg = {}
        sc = np.float32(0.1275)
        scores = (rng.standard_normal(16) * 20).astype(np.float32)
        m = np.float32(scores.max() * sc - 3.0)
        for j in range(16):
            reg[GEN.S(par, qb) + j] = int(scores[j].view(np.uint32))
        reg[GEN.NEGM + qb] = int(np.float32(-m).view(np.uint32))
        _run_valu(GEN.softmax_full(par, qb), reg, {GEN.SC: int(sc.view(np.uint32))})
        pbits = [reg[GEN.P(par, qb) + t] for t in range(8)]
        vals = []
        for w in pbits:
            vals += [np.uint32((w & 0xFFFF) << 16).view(np.float32),
                     np.uint32(w & 0xFFFF0000).view(np.float32)]
        want_bits = _bf16_rne(np.exp2(np.float32(np.float64(scores) * np.float64(sc) - np.float64(m))))
        got_bits = np.array([(w >> (16 * h)) & 0xFFFF for w in pbits for h in (0, 1)], np.uint32)
        assert np.array_equal(got_bits, want_bits)
        ps = [vals[2 * t] + vals[2 * t + 1] for t in range(8)]
        tree = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]))
        assert np.uint32(reg[GEN.LS + qb]) == np.float32(tree).view(np.uint32)


def test_checker_catches_a_sum_of_unrounded_exponentials():
    """Planted mistake: the pair sum taken from the fp32 exponentials instead of the rounded
    pair fails the block-sum check above."""
    orig = GEN.softmax_part
    def bad(par, qb, t0, t1):
        return [l for l in orig(par, qb, t0, t1)
                if not l.startswith(("v_and_b32", "v_lshlrev_b32"))]
    GEN.softmax_part = bad
    try:
        with pytest.raises(AssertionError):
            test_block_sum_is_the_sum_of_the_rounded_p()
    finally:
        GEN.softmax_part = orig


def _run_two_lanes(ops, regs, sgpr):
    """Executes the fast loop's reference-max set-up on the two lanes of one query (lane 1 is
    lane 0's partner, lane ^ 32): max3/max/mul/mov/xor per lane, ds_bpermute from the partner."""
    f = lambda reg, r: np.uint32(reg[r]).view(np.float32)
    put = lambda reg, r, x: reg.__setitem__(r, int(np.float32(x).view(np.uint32)))
    def val(reg, t):
        if t.startswith("v"):
            return f(reg, int(t[1:]))
        if t.startswith("s"):
            return np.uint32(sgpr[int(t[1:])]).view(np.float32)
        raise AssertionError(t)
    for op in ops:
        if op.startswith("s_waitcnt"):
            continue
        name, rest = op.split(None, 1)
        a = [t.strip() for t in rest.split(",")]
        d = int(a[0][1:])
        if name == "ds_bpermute_b32":
            src = int(a[2][1:])
            got = [regs[1][src], regs[0][src]]
            for lane in (0, 1):
                regs[lane][d] = got[lane]
            continue
        for reg in regs:
            if name == "v_max3_f32":
                put(reg, d, max(val(reg, a[1]), val(reg, a[2]), val(reg, a[3])))
            elif name == "v_max_f32":
                put(reg, d, max(val(reg, a[1]), val(reg, a[2])))
            elif name == "v_mul_f32":
                put(reg, d, np.float32(val(reg, a[1]) * val(reg, a[2])))
            elif name == "v_mov_b32":
                reg[d] = reg[int(a[1][1:])]
            elif name == "v_xor_b32":
                reg[d] = int(a[1], 16) ^ reg[int(a[2][1:])]
            else:
                raise AssertionError(op)


def test_fast_loop_reference_max_is_the_first_blocks_max():
    """The fast loop's prologue sets the reference max of a query block to c times the max of
    the first key block's 32 scores over both lanes of the query (and -m beside it), so the
    following softmax gives p = 1 exactly for the max key and no p above 1."""
    rng = np.random.default_rng(9)
    sc = np.float32(0.1275)
    for par, qb in ((0, 0), (0, 1)):
        for trial in range(20):
            scores = (rng.standard_normal((2, 16)) * 30).astype(np.float32)
            regs = [dict(), dict()]
            for lane in (0, 1):
                for j in range(16):
                    regs[lane][GEN.S(par, qb) + j] = int(scores[lane, j].view(np.uint32))
            sgpr = {GEN.SC: int(sc.view(np.uint32)), GEN.NINF: int(np.float32(-np.inf).view(np.uint32))}
            _run_two_lanes(GEN.init_reference_max(par, qb), regs, sgpr)
            want = np.float32(sc * scores.max())
            for lane in (0, 1):
                assert np.uint32(regs[lane][GEN.M + qb]) == want.view(np.uint32)
                assert np.uint32(regs[lane][GEN.NEGM + qb]) == (-want).view(np.uint32)
                _run_valu(GEN.softmax_full(par, qb), regs[lane], {GEN.SC: int(sc.view(np.uint32))})
                p = [np.uint32(((regs[lane][GEN.P(par, qb) + t] >> (16 * h)) & 0xFFFF) << 16).view(np.float32)
                     for t in range(8) for h in (0, 1)]
                assert max(p) <= 1.0
                if scores[lane].max() == scores.max():
                    assert max(p) == 1.0


def test_checker_catches_a_reference_max_of_one_lane():
    """Planted mistake: without the exchange with the partner lane each lane takes only its own
    16 scores' max, which the check above catches."""
    orig = GEN.init_reference_max
    def own_max(par, qb):
        out = []
        for l in orig(par, qb):
            if l.startswith("ds_bpermute_b32"):
                dst, _, src = [t.strip() for t in l.split(None, 1)[1].split(",")]
                l = f"v_mov_b32 {dst}, {src}"      # the lane's own max instead of its partner's
            out.append(l)
        return out
    GEN.init_reference_max = own_max
    try:
        with pytest.raises(AssertionError):
            test_fast_loop_reference_max_is_the_first_blocks_max()
    finally:
        GEN.init_reference_max = orig
