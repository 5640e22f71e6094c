"""Pins for the oracle's Dynamic Token Selection (score + grouping).

The pages ("Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor
Efficiënte Videogeneratie" §2.1 and the §2 introduction) fix: tokens are grouped
by the per-token L1 relative change of their velocity predictions, and the
slower-changing tokens receive the smaller budgets.  The norm ratio, the fp32
summation tree, the zero/NaN rules and the tie order are readings; the tests
below pin each of them to hand values, closed forms or brute force.
"""
import math

import numpy as np
import pytest

import oracle

F = np.float32


def test_hand_values():
    C = 16
    one = np.ones((1, C), F)
    assert oracle.l1_relative_change(one, 1.5 * one)[0] == F(0.5)
    assert oracle.l1_relative_change(one, one)[0] == F(0.0)
    assert oracle.l1_relative_change(2 * one, -2 * one)[0] == F(2.0)
    z = np.zeros((1, C), F)
    assert oracle.l1_relative_change(z, z)[0] == F(0.0)            # 0/0 -> 0
    assert oracle.l1_relative_change(z, one)[0] == F(np.inf)       # x/0 -> +inf
    nan = one.copy()
    nan[0, 3] = np.nan
    assert oracle.l1_relative_change(one, nan)[0] == F(np.inf)     # NaN -> +inf
    r = oracle.l1_relative_change(np.stack([one[0], z[0], one[0]]),
                                  np.stack([3 * one[0], z[0], one[0]]))
    assert r.tolist() == [2.0, 0.0, 0.0]


def test_tree_association():
    # [1, 1, 2^-23, 2^-23]: the balanced tree gives (1+1) + (2^-23+2^-23) = 2 + 2^-22 exactly,
    # while a left-to-right fp32 sum loses both small terms (2 + 2^-23 rounds to even: 2).
    row = np.array([[1.0, 1.0, 2.0 ** -23, 2.0 ** -23]], F)
    assert oracle.tree_sum_rows(row)[0] == F(2.0 + 2.0 ** -22)
    seq = F(0)
    for v in row[0]:
        seq = F(seq + v)
    assert seq == F(2.0)
    # the same row as a velocity change against |v_prev| = 4: r = (2 + 2^-22)/4 = 0.5 + 2^-24
    vp = np.ones((1, 4), F)
    vc = (vp + row).astype(F)
    assert oracle.l1_relative_change(vp, vc)[0] == F(0.5 + 2.0 ** -24)
    # zero padding to the next power of two: width 3 sums as (a0+a1) + (a2+0)
    row3 = np.array([[1.0, 2.0 ** -24, 2.0 ** -24]], F)
    assert oracle.tree_sum_rows(row3)[0] == F(1.0)   # (1 + 2^-24 -> 1) + 2^-24 -> 1


def butterfly_sum(row, per_lane):
    """Sum as a wavefront does it: each lane first adds its per_lane contiguous values as a
    balanced tree, then lanes combine with xor-offsets 1, 2, 4, ... (a different program
    order from the level-by-level tree; identical rounding iff the tree is balanced)."""
    C = row.shape[0]
    lanes = max(1, C // per_lane)
    vals = []
    for l in range(lanes):
        chunk = list(row[l * per_lane:(l + 1) * per_lane])
        while len(chunk) > 1:
            chunk = [F(chunk[2 * j] + chunk[2 * j + 1]) for j in range(len(chunk) // 2)]
        vals.append(chunk[0])
    off = 1
    while off < lanes:
        vals = [F(vals[l] + vals[l ^ off]) for l in range(lanes)]
        off *= 2
    assert all(v == vals[0] for v in vals)
    return vals[0]


@pytest.mark.parametrize("C", [4, 16, 64])
def test_tree_equals_butterfly(C):
    r = np.random.default_rng(C)
    x = np.abs(r.standard_normal((300, C)).astype(F) * (2.0 ** r.integers(-20, 20, (300, 1)))).astype(F)
    tree = oracle.tree_sum_rows(x)
    for n in range(x.shape[0]):
        assert tree[n] == butterfly_sum(x[n], 1)
        assert tree[n] == butterfly_sum(x[n], 4)


def test_fp64_agreement_and_scaling():
    r = np.random.default_rng(1)
    for C in (16, 64):
        vp = r.standard_normal((500, C)).astype(F)
        vc = (vp + r.lognormal(0, 1, (500, 1)).astype(F) * r.standard_normal((500, C)).astype(F)).astype(F)
        got = oracle.l1_relative_change(vp, vc)
        d = np.abs(vc.astype(np.float64) - vp.astype(np.float64))
        for n in range(500):
            exact = math.fsum(d[n]) / math.fsum(np.abs(vp[n].astype(np.float64)))
            # pairwise-sum error bound: each sum within log2(C)+1 roundings, plus the divide
            # and the fp32 subtraction: relative error well under (2*log2(C)+4) * 2^-24
            bound = (2 * math.log2(C) + 4) * 2.0 ** -24 * exact
            assert abs(float(got[n]) - exact) <= bound
        # power-of-two scaling leaves every rounding step unchanged -> bit-identical scores
        for k in (-3, 5):
            s = F(2.0 ** k)
            assert np.array_equal(oracle.l1_relative_change(vp * s, vc * s).view(np.uint32),
                                  got.view(np.uint32))


def brute_rank(r):
    n = len(r)
    key = r.view(np.uint32)
    rank = np.zeros(n, np.int64)
    for a in range(n):
        rank[a] = sum(1 for j in range(n) if key[j] > key[a]) + \
                  sum(1 for j in range(a) if key[j] == key[a])
    return rank


def test_grouping_brute_force():
    r = np.random.default_rng(2)
    for trial in range(20):
        n = int(r.integers(1, 120))
        vals = r.choice([0.0, 0.25, 0.5, 1.0, 2.0, np.inf], n) if trial % 2 else r.random(n)
        s = vals.astype(F)
        K = int(r.integers(1, 5))
        cuts = np.sort(r.integers(0, n + 1, K - 1))
        sizes = np.diff(np.concatenate([[0], cuts, [n]])).astype(np.int64)
        g = oracle.assign_groups(s, sizes)
        rank = brute_rank(s)
        bounds = np.cumsum(sizes)
        want = np.array([int(np.sum(bounds <= rk)) for rk in rank])
        assert np.array_equal(g, want)
        for k in range(K):
            assert int(np.sum(g == k)) == sizes[k]
        for k in range(K - 1):
            a, b = s[g == k], s[g == k + 1]
            if a.size and b.size:
                assert a.min() >= b.max()      # faster-changing tokens sit in earlier groups


def test_forced_ties_are_index_ordered():
    n = 37
    s = np.full(n, 0.75, F)
    g = oracle.assign_groups(s, [10, 20, 7])
    assert g.tolist() == [0] * 10 + [1] * 20 + [2] * 7


def test_largest_change_goes_to_full_budget_group():
    s = np.array([0.1, 5.0, 0.2, 3.0], F)
    g = oracle.assign_groups(s, [2, 2])
    assert g.tolist() == [1, 0, 1, 0]
