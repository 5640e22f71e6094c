"""GPU parity on seeded random configurations, beyond the hand-picked cases.

Shapes, group layouts and schedules are drawn once from a fixed seed, so every run checks
the same cases: ragged token and query counts around the tile sizes, both head sizes,
batches of one to three, group sizes that include empty groups, and schedules with and
without the full-compute window.  The bars are those of the hand-picked tests: selection,
active sets, cache rows and the Euler state bit-exact; attention within the float64
oracle's tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_l1_amd import synth
from tests.gpu_helpers import attn_close, bits_dev, dev, host, host_bits, velocities

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20261203)


def _attn_case():
    d = int(_R.choice([64, 128]))
    n = int(_R.choice([int(_R.integers(1, 300)), int(_R.integers(256, 3000))]))
    return (int(_R.integers(1, 4)), int(_R.integers(1, 700)), n, int(_R.integers(1, 4)), d,
            float(_R.choice([1.0, 1.0, 4.0])))


ATTN = [_attn_case() for _ in range(24)]


def _schedule_case():
    T = int(_R.choice([8, 12, 16, 40]))
    divisors = [s for s in range(1, T + 1) if T % s == 0]
    k = int(_R.integers(1, 6))
    budgets = sorted({T} | {int(_R.choice(divisors)) for _ in range(k - 1)}, reverse=True)
    n = int(_R.choice([int(_R.integers(1, 100)), int(_R.integers(100, 20000))]))
    cuts = np.sort(_R.integers(0, n + 1, len(budgets) - 1))
    sizes = tuple(int(x) for x in np.diff(np.concatenate([[0], cuts, [n]])))
    return (n, int(_R.integers(1, 97)), tuple(budgets), sizes, T, int(_R.integers(0, T // 2 + 1)),
            str(_R.choice(["lognormal", "heavy", "ties", "levels", "special"])))


SCHED = [_schedule_case() for _ in range(20)]


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


@pytest.mark.parametrize("case", range(len(ATTN)))
def test_attention_random(hs, case):
    B, A, N, H, D, qs = ATTN[case]
    r = np.random.default_rng(1000 + case)
    q = synth.f32_to_bf16_bits((r.standard_normal((B, A, H, D)) * qs).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    attn_close(host_bits(o), want, f"random {ATTN[case]}")
    # the workspace entry point (the sampler's): with few query tiles, most of these shapes
    # split their key ranges
    ow = torch.empty_like(o)
    hs.hsa_attention_active_ws(bits_dev(q), bits_dev(k), bits_dev(v), ow, scale,
                               hs.attention_workspace(A, N, B, H, D))
    torch.cuda.synchronize()
    attn_close(host_bits(ow), want, f"random {ATTN[case]} with workspace")


@pytest.mark.parametrize("case", range(len(SCHED)))
def test_selection_and_schedule_random(hs, case):
    n, c, budgets, sizes, T, m, kind = SCHED[case]
    vp, vc = velocities(kind, n, c, 2000 + case)
    g_want, r_want = oracle.select_groups(vp, vc, sizes)
    g = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    score = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = hs.workspace(n, len(sizes))
    hs.hsa_select_groups(dev(vp), dev(vc), sizes, g, score, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(score).view(np.uint32), r_want.view(np.uint32))
    assert np.array_equal(host(g), g_want)
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int32, device="cuda")
    for i in range(T):
        na = hs.hsa_active_set(g, budgets, sizes, T, m, i, idx, pos, ws)
        want_idx, want_pos = oracle.active_set(g_want, budgets, T, m, i)
        assert na == want_idx.shape[0] == hs.hsastep_n_active(n, budgets, sizes, T, m, i)
        assert np.array_equal(host(idx)[:na], want_idx), f"iteration {i}"
        assert np.array_equal(host(pos), want_pos), f"iteration {i}"


@pytest.mark.parametrize("case", range(12))
def test_kv_update_and_euler_random(hs, case):
    r = np.random.default_rng(3000 + case)
    B, N, H = int(r.integers(1, 4)), int(r.integers(1, 5000)), int(r.integers(1, 5))
    D = int(r.choice([64, 128]))
    C = int(r.choice([1, 3, 4, 16, 64, 68]))
    na = int(r.integers(0, N + 1))
    idx = np.sort(r.choice(N, na, replace=False)).astype(np.int32)
    kc = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    vc = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    kn = synth.f32_to_bf16_bits(r.standard_normal((B, na, H, D)).astype(np.float32))
    vn = synth.f32_to_bf16_bits(r.standard_normal((B, na, H, D)).astype(np.float32))
    kd, vd = bits_dev(kc), bits_dev(vc)
    idx_d = dev(idx) if na else dev(np.zeros(1, np.int32))
    hs.hsa_kv_update(kd, vd, bits_dev(kn), bits_dev(vn), idx_d, na)
    oracle.kv_update(kc, vc, kn, vn, idx)
    assert np.array_equal(host_bits(kd), kc)
    assert np.array_equal(host_bits(vd), vc)

    x = r.standard_normal((N, C)).astype(np.float32)
    vh = r.standard_normal((N, C)).astype(np.float32)
    pos = np.full(N, -1, np.int32)
    pos[idx] = np.arange(na, dtype=np.int32)
    vf = r.standard_normal((max(na, 1), C)).astype(np.float32)
    sig = oracle.sigma_schedule(40)
    i = int(r.integers(0, 40))
    xd, vhd = dev(x), dev(vh)
    hs.hsa_euler_step(xd, vhd, dev(vf), dev(pos), na, float(sig[i]), float(sig[i + 1]))
    xw, vw = oracle.euler_step(x, vh, vf[:na], idx, sig[i], sig[i + 1])
    assert np.array_equal(host(vhd), vw)
    assert np.array_equal(host(xd).view(np.uint32), xw.view(np.uint32))
