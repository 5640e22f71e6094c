"""Pins for the oracle's step schedule (active sets).

The schedule is fixed by "Technische Samenvatting: Heterogene Staptoewijzing (HSA)
voor Efficiënte Videogeneratie" §2.1 (budgets divide T, G_1 always active, reduced
groups active iff i mod (T/s_k) = 0) and §2.4 (full first/last m iterations).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_fractions.txt")


def load_golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        head, fr, counts, total = [p.strip() for p in line.split("|")]
        name, T, m, budgets, sizes = head.split()
        rows[name] = dict(T=int(T), m=int(m), budgets=tuple(int(b) for b in budgets.split(",")),
                          sizes=tuple(int(s) for s in sizes.split(",")),
                          fractions=None if fr == "-" else [float(f) for f in fr.split(",")],
                          counts=[int(c) for c in counts.split(",")], total=float(total))
    return rows


@pytest.mark.parametrize("name", ["tiny", "full_schedule", "aggressive_pair"])
def test_golden_fractions(name):
    row = load_golden()[name]
    T, m, budgets, sizes = row["T"], row["m"], row["budgets"], row["sizes"]
    N = sum(sizes)
    g = np.repeat(np.arange(len(sizes)), sizes).astype(np.int32)
    fr = []
    counts = np.zeros(len(sizes), int)
    for i in range(T):
        idx, _ = oracle.active_set(g, budgets, T, m, i)
        fr.append(idx.shape[0] / N)
        for k in range(len(sizes)):
            counts[k] += int(np.isin(np.flatnonzero(g == k)[:1], idx).all())
        assert idx.shape[0] == oracle.n_active(sizes, budgets, T, m, i)
    if row["fractions"] is not None:
        np.testing.assert_allclose(fr, row["fractions"])
    assert list(counts) == row["counts"]
    assert abs(sum(fr) - row["total"]) < 1e-9


def divisors(T):
    return [d for d in range(1, T + 1) if T % d == 0]


@pytest.mark.parametrize("T", [1, 2, 6, 8, 12, 40])
def test_closed_forms(T):
    # without a window, a group of budget s is active at exactly the s iterations 0, T/s, 2T/s, ...
    for s in divisors(T):
        act = [i for i in range(T) if oracle.group_active(i, s, T, 0)]
        assert act == list(range(0, T, T // s))
        assert len(act) == s
    # the baseline group (s_1 = T) is active at every iteration, for every window
    for m in range(0, T + 1):
        assert all(oracle.group_active(i, T, T, m) for i in range(T))
    # 2m >= T: every iteration is inside a window, so every group is active
    for m in range((T + 1) // 2, T + 1):
        for s in divisors(T):
            assert all(oracle.group_active(i, s, T, m) for i in range(T))
    # the window covers exactly the first and last m iterations
    for m in range(0, T // 2 + 1):
        smallest = 1
        act = [i for i in range(T) if oracle.group_active(i, smallest, T, m)]
        expect = sorted(set(range(m)) | set(range(T - m, T)) | {0})
        assert act == expect


def test_active_set_brute_force():
    r = np.random.default_rng(5)
    for _ in range(40):
        T = int(r.choice([4, 8, 12, 16, 40]))
        ds = divisors(T)
        K = int(r.integers(1, 5))
        budgets = [T] + sorted([int(r.choice(ds)) for _ in range(K - 1)], reverse=True)
        N = int(r.integers(1, 200))
        g = r.integers(0, K, N).astype(np.int32)
        m = int(r.integers(0, T // 2 + 2))
        i = int(r.integers(0, T))
        idx, pos = oracle.active_set(g, budgets, T, m, i)
        want = []
        for n in range(N):
            s = budgets[g[n]]
            if i < m or i >= T - m or i % (T // s) == 0:
                want.append(n)
        assert idx.tolist() == want
        assert idx.dtype == np.int32 and pos.dtype == np.int32
        for n in range(N):
            assert pos[n] == (want.index(n) if n in want else -1)


def test_budget_validation():
    with pytest.raises(ValueError):
        oracle.check_budgets([20, 10], 40)     # s_1 != T
    with pytest.raises(ValueError):
        oracle.check_budgets([40, 15], 40)     # 15 does not divide 40
    with pytest.raises(ValueError):
        oracle.check_budgets([], 40)
    oracle.check_budgets([40, 20, 10, 5], 40)
