"""The generated reduction loop of the fused QKV projection, checked without a GPU.

The loop is hand-scheduled assembly (proj_loop_gen.py), so the wait states between dependent
instructions, the LDS counter waits, the registers it may touch, its LDS offsets and the
bookkeeping of its stage buffers (which stage each tile load fetches, into which buffer, and
the barriers that order the four wavefronts) are checked here; a planted mistake of each kind
must be caught.
"""
import os

import pytest

import loop_checker as lc

GEN = lc.load_generator("proj_loop_gen")
HIP = open(os.path.join(lc.CSRC, "proj.hip")).read()


def test_hazards_and_lds_counters():
    assert lc.check_proj_hazards(GEN) == []


def test_registers_are_declared():
    assert lc.check_registers(GEN, HIP) == []


def test_lds_offsets_in_bounds():
    assert lc.check_proj_lds_bounds(GEN) == []


@pytest.mark.parametrize("nstage", [1, 2, 3, 4, 5, 24, 79, 80])
def test_stage_walk(nstage):
    """For every start stage rot: the t-th stage of the walk, column (rot + t) mod nstage, is
    loaded once into buffer t % 2, from inside the rows, and read once per k-step (two), in
    order; the last group of reads (the next stage's k-step 0, after the end) reads the
    empty-range loads and is unused."""
    rots = range(nstage) if nstage < 30 else (0, 1, nstage // 2, nstage - 2, nstage - 1)
    for rot in rots:
        ksteps, errors = lc.proj_stage_walk(GEN, nstage, rot=rot)
        assert errors == [], (rot, errors[:3])
        assert ksteps[:-1] == [(rot + t) % nstage for t in range(nstage) for _ in range(GEN.KSTEPS)]
        assert ksteps[-1] is None


def test_loop_shape():
    body = GEN.generate()
    loop = body[body.index(".Lploop:"):body.index("s_branch .Lploop")]
    assert sum(l.startswith("v_mfma") for l in loop) == 2 * 128       # two stages of 2 x 64
    assert sum(l == "s_barrier" for l in loop) == 2                   # one per stage
    assert sum(l.startswith("buffer_load") for l in loop) == 2 * 16
    assert sum(l.startswith("ds_read_b128") for l in loop) == 2 * 32


def _patched(name, fn, check):
    orig = getattr(GEN, name)
    setattr(GEN, name, fn(orig))
    try:
        return check()
    finally:
        setattr(GEN, name, orig)


def _walk_errors():
    return [e for n in (2, 3, 5) for e in lc.proj_stage_walk(GEN, n)[1]]


def test_walk_catches_a_missing_barrier():
    errs = _patched("stage", lambda f: lambda par: [l for l in f(par) if l != "s_barrier"],
                    _walk_errors)
    assert any("no barrier" in e for e in errs)


def test_walk_catches_a_missing_load_wait():
    errs = _patched("stage", lambda f: lambda par: [l.replace("vmcnt(0) ", "") for l in f(par)],
                    _walk_errors)
    assert any("incomplete" in e or "still loads" in e for e in errs)


def test_walk_catches_a_missing_wrap():
    """Without the move back at the wrap point the loads run past the end of the rows."""
    def nowrap(f):
        return lambda ahead: [l for l in f(ahead) if not l.startswith("s_sub")]
    errs = _patched("advance", nowrap,
                    lambda: [e for n in (3, 5) for e in lc.proj_stage_walk(GEN, n, rot=2)[1]])
    assert any("outside the rows" in e for e in errs)


def test_walk_catches_a_wrong_descriptor_advance():
    errs = _patched("advance", lambda f: lambda ahead: f(ahead) + f(ahead)[:4], _walk_errors)
    assert any("loaded as" in e for e in errs)


def test_checker_catches_a_missing_lds_wait():
    errs = _patched("stage", lambda f: lambda par: [l for l in f(par) if l != "s_waitcnt lgkmcnt(0)"],
                    lambda: lc.check_proj_hazards(GEN))
    assert any("LDS result is in flight" in e for e in errs)


def test_checker_catches_an_early_accumulator_read():
    # a VALU read of an accumulator right after the MFMA that writes it
    def early(f):
        def g(par):
            out = f(par)
            i = next(k for k, l in enumerate(out) if l.startswith("v_mfma"))
            return out[:i + 1] + ["v_accvgpr_read_b32 v0, a0"] + out[i + 1:]
        return g
    errs = _patched("stage", early, lambda: lc.check_proj_hazards(GEN))
    assert any("needs 12" in e for e in errs)


def test_checker_catches_an_undeclared_register():
    orig = GEN.clobbered
    GEN.clobbered = lambda: {k: (s - {40} if k == "v" else s) for k, s in orig().items()}
    try:
        assert any("('v', 40)" in e for e in lc.check_registers(GEN, HIP))
    finally:
        GEN.clobbered = orig
