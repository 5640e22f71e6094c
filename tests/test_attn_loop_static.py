"""The generated key loop of the head_dim 128 attention kernel, checked without a GPU.

The loop is hand-scheduled assembly (attn_loop_gen.py), so the wait states the hardware needs
between dependent instructions, the LDS counter waits, the registers it may touch and its LDS
offsets are checked here statically; a planted mistake of each kind must be caught.
"""
import os

import pytest

import loop_checker as lc

GEN = lc.load_generator()
HIP = open(os.path.join(lc.CSRC, "attn_pipe.hip")).read()


def test_hazards_and_lds_counters():
    assert lc.check_hazards(GEN) == []


def test_registers_are_declared():
    assert lc.check_registers(GEN, HIP) == []


def test_lds_offsets_in_bounds():
    assert lc.check_lds_bounds(GEN) == []


def test_loop_shape():
    body = GEN.generate()
    mf = [l for l in body if l.startswith("v_mfma")]
    # per step: 16 S^T MFMAs (two chains of 8), 16 P.V MFMAs, and two row-sum MFMAs for each
    # of the two blocks whose softmax ends in the step; 8 unrolled steps
    loop = body[body.index(".Lloop:"):body.index("s_branch .Lloop")]
    assert sum(l.startswith("v_mfma_f32_32x32x16_bf16") for l in loop) == 8 * 32
    assert sum(l.startswith("v_mfma_f32_16x16x32_bf16") for l in loop) == 8 * 4
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
    errs = _with_patch("step", lambda f: lambda r: [l for l in f(r) if "lgkmcnt(8)" not in l])
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
        def g(r):
            out = f(r)
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


def test_checker_catches_an_early_block_sum_read():
    # the range check reading a block sum before its row-sum MFMA has finished
    def early(f):
        def g(r):
            out = f(r)
            i = out.index("s_nop 3")
            return out[:i - 1] + out[i + 1:]
        return g
    errs = _with_patch("step", early)
    assert any("needs 12" in e for e in errs)


def test_row_sum_operand_pattern():
    """The A operand of the row-sum MFMA (lane l holds ones iff bit 2 of l equals bit 4) makes
    every lane's result its own query's sum over the block's 32 keys.  Checked with the
    16x16x32 operand layouts (A: lane l row l%16, k-group l/16; B: lane l column l%16, k-group
    l/16; result: lane l column l%16, rows 4(l/16)..+3) and the S^T layout (lane q + 32g holds
    query q)."""
    import numpy as np
    rng = np.random.default_rng(0)
    lane = np.arange(64)
    ones = (((lane >> 2) & 1) == ((lane >> 4) & 1)).astype(np.float64)
    pvals = rng.random((64, 8))                # 8 packed P values held by each lane
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for l in range(64):
        A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = ones[l]
        B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = pvals[l]
    D = A @ B
    query = lane % 32                           # S^T accumulator: lane q + 32g holds query q
    want = np.array([pvals[query == q].sum() for q in range(32)])
    for l in range(64):
        got = D[4 * (l // 16):4 * (l // 16) + 4, l % 16]
        assert np.allclose(got, want[query[l]])
