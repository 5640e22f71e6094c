"""Host-side checks of the C ABI (no GPU needed).

The library must load on a GPU-less host, export exactly the functions that
include/hsastep.h declares, and reject invalid arguments on the host before
anything reaches the device.  The closed-form |A_i| is compared with the
oracle's brute-force schedule.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsastep.h")
LIB = os.path.join(ROOT, "sparse_attention_l1_amd", "libhsastep.so")


@pytest.fixture(scope="module")
def hs():
    if not os.path.exists(LIB):
        from sparse_attention_l1_amd import build
        build.build()
    from sparse_attention_l1_amd import hsastep
    return hsastep


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:hsa|hsastep)_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(hs):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l})
    ours = [e for e in exported if e.startswith(("hsa_", "hsastep_"))]
    assert ours == declared_functions()
    # nothing else of ours leaks (hidden visibility); no symbol may shadow the ROCm HSA runtime
    assert not any(e.startswith("hsa_status") for e in exported)
    assert set(hs.EXPORTED) == set(declared_functions())


def test_version_and_strings(hs):
    assert hs.hsastep_version() >= 100
    assert hs.lib.hsastep_error_string(-1) == b"invalid argument"
    assert hs.lib.hsastep_error_string(0) == b"ok"


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first


def call(hs, name, *args):
    return getattr(hs.lib, name)(*args)


def test_select_groups_rejects(hs):
    sizes = (ctypes.c_int64 * 2)(5, 5)
    bad_sizes = (ctypes.c_int64 * 2)(5, 4)
    neg = (ctypes.c_int64 * 2)(11, -1)
    ws = hs.hsastep_workspace_bytes(10, 2)
    f = lambda *a: call(hs, "hsa_select_groups", *a)
    assert f(FAKE, FAKE, 10, 16, bad_sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 10, 16, neg, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 0, 16, sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 10, 0, sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 10, 257, sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 10, 16, sizes, 17, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(None, FAKE, 10, 16, sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert f(ctypes.c_void_p((1 << 20) + 4), FAKE, 10, 16, sizes, 2, FAKE, FAKE, FAKE, ws,
             None) == hs.ERR_ARG
    # no / too small workspace, with or without a score output
    assert f(FAKE, FAKE, 10, 16, sizes, 2, FAKE, None, None, 0, None) == hs.ERR_WORKSPACE
    assert f(FAKE, FAKE, 10, 16, sizes, 2, FAKE, FAKE, None, ws, None) == hs.ERR_WORKSPACE
    assert f(FAKE, FAKE, 10, 16, sizes, 2, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 8), ws,
             None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 10, 16, sizes, 2, FAKE, None, FAKE, ws - 1, None) == hs.ERR_WORKSPACE
    assert f(FAKE, FAKE, 10, 16, bad_sizes, 2, FAKE, FAKE, FAKE, ws, None) == hs.ERR_ARG
    assert b"sum to n_tokens" in hs.lib.hsastep_last_error()


def test_active_set_rejects(hs):
    def run(budgets, sizes, T, m, it, n=None, ws=None):
        b = (ctypes.c_int32 * len(budgets))(*budgets)
        s = (ctypes.c_int64 * len(sizes))(*sizes)
        n = sum(sizes) if n is None else n
        out = ctypes.c_int64(-7)
        w = hs.hsastep_workspace_bytes(max(n, 1), len(budgets)) if ws is None else ws
        return call(hs, "hsa_active_set", FAKE, n, b, s, len(budgets), T, m, it, FAKE, FAKE,
                    ctypes.byref(out), FAKE, w, None)
    assert run([20, 10], [5, 5], 40, 4, 5) == hs.ERR_ARG       # s_1 != T
    assert run([40, 15], [5, 5], 40, 4, 5) == hs.ERR_ARG       # 15 does not divide 40
    assert run([40, 5, 10], [3, 3, 4], 40, 4, 5) == hs.ERR_ARG  # not non-increasing
    assert run([40, 20], [5, 4], 40, 4, 5, n=10) == hs.ERR_ARG  # sizes do not sum to N
    assert run([40, 20], [5, 5], 40, -1, 5) == hs.ERR_ARG      # m < 0
    assert run([40, 20], [5, 5], 40, 4, 40) == hs.ERR_ARG      # iter >= T
    assert run([40, 20], [5, 5], 40, 4, -1) == hs.ERR_ARG
    assert run([40, 20], [5, 5], 40, 4, 5, ws=16) == hs.ERR_WORKSPACE
    assert run([40, 15], [5, 5], 40, 4, 5) == hs.ERR_ARG
    assert b"divide" in hs.lib.hsastep_last_error()


def test_active_set_gather_rejects_on_the_host(hs):
    b = (ctypes.c_int32 * 2)(40, 20)
    sz = (ctypes.c_int64 * 2)(5, 5)
    out = ctypes.c_int64(-7)
    w = hs.hsastep_workspace_bytes(10, 2)
    run = lambda rows, rb, rows_out, ws=w: call(hs, "hsa_active_set_gather", FAKE, 10, b, sz, 2,
                                                40, 4, 5, FAKE, FAKE, ctypes.byref(out), rows, rb,
                                                rows_out, FAKE, ws, None)
    assert run(FAKE, 6, FAKE) == hs.ERR_ARG                      # row_bytes not a multiple of 4
    assert run(FAKE, 0, FAKE) == hs.ERR_ARG
    assert run(None, 16, FAKE) == hs.ERR_ARG
    assert run(FAKE, 16, ctypes.c_void_p((1 << 20) + 2)) == hs.ERR_ARG   # misaligned
    assert run(FAKE, 16, FAKE, ws=8) == hs.ERR_WORKSPACE


def test_active_set_noalloc_rejects_on_the_host(hs):
    """Validation of the allocation-free variant runs before it looks up its scratch array
    or enqueues anything: schedule errors, more tokens than the array covers, null pointers."""
    def run(budgets, sizes, T, m, it, n=None, idx=FAKE):
        b = (ctypes.c_int32 * len(budgets))(*budgets)
        s = (ctypes.c_int64 * len(sizes))(*sizes)
        n = sum(sizes) if n is None else n
        out = ctypes.c_int64(-7)
        return call(hs, "hsa_active_set_noalloc", FAKE, n, b, s, len(budgets), T, m, it, idx,
                    FAKE, ctypes.byref(out), None)
    assert run([40, 15], [5, 5], 40, 4, 5) == hs.ERR_ARG        # 15 does not divide 40
    assert run([40, 20], [5, 5], 40, 4, 40) == hs.ERR_ARG       # iter >= T
    assert run([40, 20], [5, 5], 40, 4, 5, idx=None) == hs.ERR_ARG
    big = hs.NOALLOC_MAX_TOKENS + 1
    assert run([40, 20], [big - 5, 5], 40, 4, 5) == hs.ERR_UNSUPPORTED
    assert b"HSASTEP_NOALLOC_MAX_TOKENS" in hs.lib.hsastep_last_error()


def test_kv_attention_euler_gather_reject(hs):
    kv = lambda *a: call(hs, "hsa_kv_update", *a)
    assert kv(FAKE, FAKE, FAKE, FAKE, FAKE, 5, 4, 1, 2, 64, None) == hs.ERR_ARG   # n_active > N
    assert kv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 1, 1, 3, None) == hs.ERR_ARG    # H*D % 8
    assert kv(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 1, 2, 64, None) == hs.OK        # no-op
    att = lambda *a: call(hs, "hsa_attention_active", *a)
    assert att(FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 96, 0.1, None) == hs.ERR_UNSUPPORTED
    assert att(FAKE, FAKE, FAKE, FAKE, 4, 0, 1, 2, 64, 0.1, None) == hs.ERR_ARG
    assert att(FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64, 0.0, None) == hs.ERR_ARG
    assert att(FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64, float("nan"), None) == hs.ERR_ARG
    assert att(FAKE, FAKE, FAKE, FAKE, 4, 8, 0, 2, 64, 0.1, None) == hs.ERR_ARG
    assert att(None, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64, 0.1, None) == hs.ERR_ARG
    assert att(None, None, None, None, 0, 8, 1, 2, 64, 0.1, None) == hs.OK        # no-op
    eu = lambda *a: call(hs, "hsa_euler_step", *a)
    assert eu(FAKE, FAKE, FAKE, FAKE, 5, 4, 8, 1.0, 0.9, None) == hs.ERR_ARG
    assert eu(FAKE, FAKE, FAKE, FAKE, 1, 4, 0, 1.0, 0.9, None) == hs.ERR_ARG
    assert eu(None, FAKE, FAKE, FAKE, 1, 4, 8, 1.0, 0.9, None) == hs.ERR_ARG
    ga = lambda *a: call(hs, "hsastep_gather_rows", *a)
    assert ga(FAKE, FAKE, FAKE, 4, 8, 6, None) == hs.ERR_ARG                       # row_bytes % 4
    assert ga(FAKE, FAKE, FAKE, -1, 8, 8, None) == hs.ERR_ARG
    assert ga(None, None, None, 0, 8, 8, None) == hs.OK


def test_mfma_probe_rejects(hs):
    f = lambda *a: call(hs, "hsastep_mfma_probe", *a)
    assert f(None, FAKE, 1, 1, None) == hs.ERR_ARG
    assert f(FAKE, None, 1, 1, None) == hs.ERR_ARG
    assert f(ctypes.c_void_p((1 << 20) + 2), FAKE, 1, 1, None) == hs.ERR_ARG     # misaligned
    assert f(FAKE, FAKE, 0, 1, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, (1 << 24) + 1, 1, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 1, 0, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, 1, (1 << 20) + 1, None) == hs.ERR_ARG


def test_qkv_project_rejects(hs):
    f = lambda *a: call(hs, "hsa_qkv_project", *a)
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64, 96, None) == hs.ERR_UNSUPPORTED
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 9, 8, 1, 2, 64, 64, None) == hs.ERR_ARG
    assert f(None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64, 64, None) == hs.ERR_ARG
    assert f(ctypes.c_void_p((1 << 20) + 2), FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 64,
             64, None) == hs.ERR_ARG
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, 1 << 21, 1, 16, 128, 4096,
             None) == hs.ERR_UNSUPPORTED                            # x_active above 4 GiB
    assert f(None, None, None, None, None, None, None, 0, 8, 1, 2, 64, 64, None) == hs.OK


def test_n_active_closed_form_matches_oracle(hs):
    r = np.random.default_rng(11)
    for T in (1, 4, 8, 12, 40):
        ds = [d for d in range(1, T + 1) if T % d == 0]
        for _ in range(25):
            K = int(r.integers(1, 6))
            budgets = [T] + sorted((int(r.choice(ds)) for _ in range(K - 1)), reverse=True)
            sizes = [int(x) for x in r.integers(0, 50, K)]
            N = sum(sizes)
            if N == 0:
                continue
            g = np.repeat(np.arange(K), sizes).astype(np.int32)
            for m in range(0, T // 2 + 2):
                for i in range(T):
                    want = oracle.active_set(g, budgets, T, m, i)[0].shape[0]
                    assert hs.hsastep_n_active(N, budgets, sizes, T, m, i) == want


def test_workspace_size_monotone(hs):
    a = hs.hsastep_workspace_bytes(1000, 4)
    b = hs.hsastep_workspace_bytes(100000, 4)
    assert 0 < a < b
    assert hs.hsastep_workspace_bytes(75600, 16) >= 75600 * 4 + 4 * (75600 // 1024)


def test_attention_plan(hs):
    """The split planner of hsa_attention_active_ws on a 256-CU device, for the workloads'
    shapes: whole rounds are never split; a half-empty last round is split so that its work
    spreads over the chip; the workspace bounds the plan."""
    ws = lambda a, n, b, h: hs.hsastep_attention_workspace_bytes(a, n, b, h, 128)
    plan = lambda a, n, b, h, w=None: hs.hsastep_attention_plan(
        a, n, b, h, 128, 256, ws(a, n, b, h) if w is None else w)
    assert plan(16380, 32760, 1, 12) == (768, 0, 1, 0)            # 3 whole rounds
    assert plan(32760, 32760, 1, 12) == (1536, 0, 1, 0)           # 6 whole rounds
    full, tail, s, keys = plan(8190, 32760, 1, 12)                 # 384 tiles = 1.5 rounds
    assert (full, tail) == (256, 128) and s >= 2 and 128 * s <= 512
    assert (s - 1) * keys < 32760 <= s * keys and keys % 32 == 0
    full, tail, s, keys = plan(7560, 75600, 2, 40)                 # 2400 tiles = 9.4 rounds
    assert (full, tail) == (2304, 96) and 96 * s <= 512 and s > 1
    assert plan(300, 3000, 2, 3)[1:3] == (12, 8)                   # all tiles split, 8 ranges
    assert plan(300, 3000, 2, 3, w=0) == (12, 0, 1, 0)             # no workspace: no split
    piece = ws(300, 3000, 2, 3) // 96
    assert plan(300, 3000, 2, 3, w=piece * 24)[1:3] == (12, 2)     # room for 24 pieces
    assert plan(300, 3000, 2, 3, w=piece * 24)[3] == 1504
    assert hs.hsastep_attention_plan(300, 3000, 2, 3, 64, 256, 10 ** 9) == (0, 0, 0, 0)
    assert hs.hsastep_attention_plan(300, 200, 2, 3, 128, 256, 10 ** 9) == (0, 0, 0, 0)
    for a, n in ((70, 1275), (513, 700), (1100, 20000)):
        full, tail, s, keys = plan(a, n, 2, 40)
        if s > 1:
            assert n - (s - 1) * keys >= 256                       # every range >= 8 blocks


def test_attention_plan_invariants(hs):
    """The planner on 3000 seeded random shapes, device sizes and workspaces: whole rounds stay
    whole, only a partly filled last round is split, every key range is at least 8 key blocks
    and a multiple of 32 keys, the ranges cover all keys, the pieces fit the workspace and the
    512-piece limit, and a split never lengthens the launch (in whole-tile units)."""
    r = np.random.default_rng(77)
    piece = hs.hsastep_attention_workspace_bytes(256 * 64, 4096, 1, 1, 128) // 512  # 64 tiles x 8 > 512
    for _ in range(3000):
        a = int(r.integers(1, 200001)) if r.random() < 0.5 else int(r.integers(1, 3000))
        n = int(r.integers(256, 200001))
        b, h = int(r.integers(1, 4)), int(r.integers(1, 65))
        cus = int(r.choice([8, 64, 80, 120, 256, 304]))
        full_ws = hs.hsastep_attention_workspace_bytes(a, n, b, h, 128)
        w = int(r.choice([0, full_ws, int(full_ws * r.random())]))
        full, tail, s, keys = hs.hsastep_attention_plan(a, n, b, h, 128, cus, w)
        tiles = -(-a // 256) * h * b
        if s == 1:
            assert (full, tail, keys) == (tiles, 0, 0), (a, n, b, h, cus, w)
            continue
        assert w > 0 and 2 <= s <= 8
        assert full + tail == tiles and full % cus == 0 and 0 < tail < cus
        assert tail * s <= 512 and tail * s * piece <= w
        assert keys % 32 == 0 and keys >= 256
        assert (s - 1) * keys < n <= s * keys and n - (s - 1) * keys >= 256
        assert full // cus + -(-tail * s // cus) / s <= -(-tiles // cus)
