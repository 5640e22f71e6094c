"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Bars: group ids, scores, active index lists, cache rows and the Euler state are
bit-exact; attention (bf16 in/out, fp32 accumulation) is within max-abs 2e-2 of
the float64 oracle for every input, peaky softmaxes included.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_l1_amd import synth
from tests.gpu_helpers import (SyntheticModel, attn_close, bf16_to_f64, bits_dev, dev, host,
                                host_bits, velocities)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


# ----------------------------------------------------------------------------- selection

SELECT_CASES = [
    ("lognormal", 256, 16, (128, 128)),
    ("lognormal", 1000, 64, (250, 250, 250, 250)),
    ("lognormal", 1, 64, (1,)),
    ("lognormal", 5, 3, (2, 0, 3)),
    ("special", 3001, 64, (1000, 1, 0, 2000)),
    ("ties", 2500, 16, (700, 1100, 700)),
    ("heavy", 75600, 64, (7560, 22680, 45360)),
    ("lognormal", 32760, 64, (16380, 16380)),
    ("ties", 20000, 4, (3000, 9000, 8000)),
    # more than 512 chunks of 512 tokens: workgroups then hold 2560 tokens each
    ("levels", 1100000, 1, (100000, 350000, 0, 650000)),
    ("lognormal", 4097, 255, tuple([256] * 15 + [257])),
    ("lognormal", 333, 1, (100, 233)),
]


@pytest.mark.parametrize("kind,n,c,sizes", SELECT_CASES)
def test_select_groups(hs, kind, n, c, sizes):
    vp, vc = velocities(kind, n, c, n + c)
    g_want, r_want = oracle.select_groups(vp, vc, sizes)
    g = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    r = torch.empty(n, dtype=torch.float32, device="cuda")
    hs.hsa_select_groups(dev(vp), dev(vc), sizes, g, r, hs.workspace(n, len(sizes)))
    # the workspace variant (no score output) gives the same groups
    g2 = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    hs.hsa_select_groups(dev(vp), dev(vc), sizes, g2, None, hs.workspace(n, len(sizes)))
    torch.cuda.synchronize()
    assert np.array_equal(host(r).view(np.uint32), r_want.view(np.uint32))
    assert np.array_equal(host(g), g_want)
    assert np.array_equal(host(g2), g_want)


# ----------------------------------------------------------------------------- active set

@pytest.mark.parametrize("T,m,budgets,sizes", [
    (8, 1, (8, 4), (128, 128)),
    (40, 4, (40, 20, 10, 5), (8190,) * 4),
    (40, 2, (40, 10, 5), (7560, 22680, 45360)),
    (12, 0, (12, 6, 3, 1), (1, 0, 1500, 3)),
    (6, 3, (6, 2), (10, 10)),          # 2m >= T: always dense
])
def test_active_set(hs, T, m, budgets, sizes):
    n = sum(sizes)
    rng = np.random.default_rng(n)
    g_host = rng.permutation(np.repeat(np.arange(len(sizes)), sizes)).astype(np.int32)
    g = dev(g_host)
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int32, device="cuda")
    ws = hs.workspace(n, len(budgets))
    for i in range(T):
        idx.fill_(-9)
        na = hs.hsa_active_set(g, budgets, sizes, T, m, i, idx, pos, ws)
        want_idx, want_pos = oracle.active_set(g_host, budgets, T, m, i)
        assert na == want_idx.shape[0]
        hi = host(idx)
        assert np.array_equal(hi[:na], want_idx)
        assert np.all(hi[na:] == -9)          # nothing written past |A_i|
        assert np.array_equal(host(pos), want_pos)


# ----------------------------------------------------------------------------- rows

@pytest.mark.parametrize("rows,c", [(1000, 64), (37, 3), (1, 16)])
def test_gather_rows(hs, rows, c):
    r = np.random.default_rng(rows)
    src = r.standard_normal((rows, c)).astype(np.float32)
    index = r.integers(0, rows, rows + 5).astype(np.int32)
    index[2] = rows + 3           # out of range -> zero row
    index[3] = -1
    dst = torch.full((rows + 5, c), 7.0, dtype=torch.float32, device="cuda")
    hs.hsastep_gather_rows(dst, dev(src), dev(index), rows + 5)
    want = np.where(((index >= 0) & (index < rows))[:, None], src[np.clip(index, 0, rows - 1)], 0)
    assert np.array_equal(host(dst), want.astype(np.float32))


@pytest.mark.parametrize("B,N,H,D,frac", [(2, 300, 3, 64, 0.3), (1, 32760, 12, 128, 0.5),
                                          (1, 129, 1, 128, 1.0), (1, 50, 2, 64, 0.0)])
def test_kv_update(hs, B, N, H, D, frac):
    r = np.random.default_rng(N)
    na = int(round(frac * N))
    idx = np.sort(r.choice(N, na, replace=False)).astype(np.int32)
    kc = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    vc = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    kn = synth.f32_to_bf16_bits(r.standard_normal((B, na, H, D)).astype(np.float32))
    vn = synth.f32_to_bf16_bits(r.standard_normal((B, na, H, D)).astype(np.float32))
    kd, vd = bits_dev(kc), bits_dev(vc)
    hs.hsa_kv_update(kd, vd, bits_dev(kn), bits_dev(vn), dev(idx) if na else dev(np.zeros(1, np.int32)), na)
    oracle.kv_update(kc, vc, kn, vn, idx)
    assert np.array_equal(host_bits(kd), kc)
    assert np.array_equal(host_bits(vd), vc)


# ----------------------------------------------------------------------------- attention

ATTN_CASES = [
    # B, A, N, H, D, q_scale
    (1, 300, 1000, 3, 128, 1.0),
    (2, 77, 257, 2, 64, 1.0),
    (1, 1, 1, 1, 128, 1.0),
    (1, 128, 64, 2, 64, 1.0),
    (1, 129, 65, 1, 128, 1.0),
    (1, 256, 4096, 2, 128, 1.0),
    (1, 200, 700, 2, 128, 8.0),     # peaky softmax
    (1, 200, 700, 2, 64, 16.0),     # very peaky
    (2, 40, 3000, 5, 128, 1.0),
    # head_dim 128 with N >= 256 takes the hand-scheduled kernel (attn_pipe.hip); N = 251 the
    # other one.  N = 32 nb - 5 for nb = 9..16 ends the key loop at each of its 8 unrolled
    # steps, with a ragged last block; N = 257 leaves one key in the last block.
    (1, 70, 251, 1, 128, 1.0),
    (1, 70, 256, 1, 128, 1.0),
    (1, 70, 257, 2, 128, 1.0),
] + [(1, 70, 32 * nb - 5, 1, 128, 1.0) for nb in range(9, 17)] + [
    (1, 1, 600, 1, 128, 1.0),       # one query: one wavefront with work, three without
    (1, 257, 1000, 1, 128, 1.0),    # a second query tile holding one query
    (1, 100, 900, 2, 128, 16.0),    # very peaky
    (1, 64, 2000, 40, 128, 1.0),    # 40 heads (token stride 10 KB)
    (2, 130, 5000, 2, 128, 8.0),    # peaky, both kernels' batch path
    (1, 64, 4000, 3, 64, 16.0),     # very peaky, head_dim 64
    (1, 300, 32760, 1, 128, 16.0),  # very peaky over the single-step key count
    (1, 100, 3000, 2, 128, 32.0),   # one key dominates almost every query
    (1, 100, 200, 2, 128, 32.0),    # the same on the short-cache kernel
]


@pytest.mark.parametrize("B,A,N,H,D,qs", ATTN_CASES)
def test_attention(hs, B, A, N, H, D, qs):
    r = np.random.default_rng(A * 7 + N)
    q = synth.f32_to_bf16_bits((r.standard_normal((B, A, H, D)) * qs).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    # output with a guard band of extra rows that must stay untouched
    out = torch.full((B * A * H * D + 4096,), 0x7F7F, dtype=torch.int16, device="cuda")
    o = out[: B * A * H * D].view(B, A, H, D)
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    attn_close(host_bits(o), want, f"B{B} A{A} N{N} H{H} D{D} x{qs}")
    assert bool((out[B * A * H * D:] == 0x7F7F).all())
    # determinism, and independence of a query from its tile neighbours
    o2 = torch.empty_like(o)
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o2, scale)
    assert torch.equal(o, o2)
    sub = np.arange(0, A, 3)
    o3 = torch.empty((B, sub.size, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q[:, sub]), bits_dev(k), bits_dev(v), o3, scale)
    assert np.array_equal(host_bits(o3), host_bits(o)[:, sub])


@pytest.mark.parametrize("N,D,late", [(2000, 128, (1500,)), (2000, 128, (1500, 1999)),
                                       (700, 64, (650,))])
def test_attention_late_outlier_key(hs, N, D, late):
    """Keys far above every earlier score: 2^(s c - m) against the earlier reference max
    would overflow fp32 (s c - m is about 400 in log2 units), so the kernels must move the
    reference before using these keys; the output is the mean of the outliers' values."""
    B, A, H = 1, 100, 2
    r = np.random.default_rng(N + D)
    qf = r.standard_normal((B, A, H, D)).astype(np.float32)
    kf = r.standard_normal((B, N, H, D)).astype(np.float32)
    qf[..., 0] = 40.0
    kf[..., 0] = 0.0
    for j in late:
        kf[:, j, :, 0] = 80.0
    q, k = synth.f32_to_bf16_bits(qf), synth.f32_to_bf16_bits(kf)
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    attn_close(host_bits(o), want, f"outlier N{N} D{D} {late}")
    assert not np.isnan(bf16_to_f64(host_bits(o))).any()


@pytest.mark.parametrize("N", [1000, 5000])
def test_attention_fallback_per_query(hs, N):
    """Every third query meets keys about 400 (base 2) above its first key block's max, so
    p against that block's reference would overflow fp32: those queries leave the fast body
    out of range and are redone by the checked body, while their tile neighbours keep the fast
    result.  Against the oracle, the bits of a query do not depend on its neighbours (a launch
    of every second query gives the same rows), and the same holds through the split path."""
    B, A, H, D = 1, 300, 2, 128
    r = np.random.default_rng(N + 5)
    qf = r.standard_normal((B, A, H, D)).astype(np.float32)
    kf = r.standard_normal((B, N, H, D)).astype(np.float32)
    qf[:, ::3, :, 0] = 40.0
    kf[:, :, :, 0] = 0.0
    for j in (N // 2, N - 37):
        kf[:, j, :, 0] = 80.0
    q, k = synth.f32_to_bf16_bits(qf), synth.f32_to_bf16_bits(kf)
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    attn_close(host_bits(o), want, f"fallback per query N{N}")
    sub = np.arange(0, A, 2)
    o2 = torch.empty((B, sub.size, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q[:, sub]), bits_dev(k), bits_dev(v), o2, scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o2), host_bits(o)[:, sub])
    ws = hs.attention_workspace(A, N, B, H, D)
    o3 = torch.empty_like(o)
    hs.hsa_attention_active_ws(bits_dev(q), bits_dev(k), bits_dev(v), o3, scale, ws)
    torch.cuda.synchronize()
    attn_close(host_bits(o3), want, f"fallback per query, split, N{N}")


@pytest.mark.parametrize("N", [1000, 1009, 4097])
def test_attention_ragged_last_block(hs, N):
    """The fast loop does not mask the keys past the end of a ragged last block; it takes their
    p back out of the row sum.  Every second query here has a negative first-block max (its
    keys 0..31 point away from it), so a padded key's p would exceed 1: those queries go to the
    checked loop, which masks, and the rest keep the fast loop's corrected sum.  Against the
    oracle, also through the split path, and a query's bits do not depend on its neighbours."""
    B, A, H, D = 1, 300, 2, 128
    r = np.random.default_rng(N + 11)
    qf = r.standard_normal((B, A, H, D)).astype(np.float32)
    kf = r.standard_normal((B, N, H, D)).astype(np.float32)
    qf[:, ::2, :, 0] = -8.0
    kf[:, :32, :, 0] = 8.0
    q, k = synth.f32_to_bf16_bits(qf), synth.f32_to_bf16_bits(kf)
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    attn_close(host_bits(o), want, f"ragged last block N{N}")
    sub = np.arange(1, A, 2)
    o2 = torch.empty((B, sub.size, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q[:, sub]), bits_dev(k), bits_dev(v), o2, scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o2), host_bits(o)[:, sub])
    ws = hs.attention_workspace(A, N, B, H, D)
    o3 = torch.empty_like(o)
    hs.hsa_attention_active_ws(bits_dev(q), bits_dev(k), bits_dev(v), o3, scale, ws)
    torch.cuda.synchronize()
    attn_close(host_bits(o3), want, f"ragged last block, split, N{N}")


def test_attention_every_last_block_width(hs):
    """Every width of the last key block, 1 to 32 keys (N = 257 .. 288), with half of the
    queries on the fast loop's corrected row sum and half (negative first-block max) on the
    checked loop, against the oracle."""
    B, A, H, D = 1, 96, 2, 128
    scale = float(np.float32(1.0 / np.sqrt(D)))
    for N in range(257, 289):
        r = np.random.default_rng(N)
        qf = r.standard_normal((B, A, H, D)).astype(np.float32)
        kf = r.standard_normal((B, N, H, D)).astype(np.float32)
        qf[:, 1::2, :, 0] = -8.0
        kf[:, :32, :, 0] = 8.0
        q, k = synth.f32_to_bf16_bits(qf), synth.f32_to_bf16_bits(kf)
        v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
        o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
        hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
        torch.cuda.synchronize()
        attn_close(host_bits(o), oracle.attention_active(q, k, v, scale), f"last block of {N - 256} keys")


@pytest.mark.parametrize("D,N,key", [(128, 1000, 3), (128, 1000, 700), (64, 500, 300)])
def test_attention_nan_key(hs, D, N, key):
    """A NaN in one cached key of head 1 makes every score of that head NaN, so the oracle's
    softmax is NaN for all of head 1's queries; the kernels give NaN there too (a NaN row sum
    also sends the fast loop's queries to the checked loop), and head 0 is unaffected."""
    B, A, H = 1, 300, 2
    r = np.random.default_rng(N + key)
    q = synth.f32_to_bf16_bits(r.standard_normal((B, A, H, D)).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    k[0, key, 1, 5] = 0x7FC0                      # a quiet NaN in bf16
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    want = oracle.attention_active(q, k, v, scale)
    assert np.isnan(want[:, :, 1]).all() and np.isfinite(want[:, :, 0]).all()
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(q), bits_dev(k), bits_dev(v), o, scale)
    torch.cuda.synchronize()
    got = bf16_to_f64(host_bits(o))
    assert np.isnan(got[:, :, 1]).all()
    attn_close(host_bits(o)[:, :, :1], want[:, :, :1], f"NaN key D{D} N{N} key {key}, head 0")


def test_attention_zero_query_is_mean(hs):
    B, A, N, H, D = 1, 5, 999, 2, 128
    r = np.random.default_rng(1)
    k = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, D)).astype(np.float32))
    o = torch.empty((B, A, H, D), dtype=torch.int16, device="cuda")
    hs.hsa_attention_active(bits_dev(np.zeros((B, A, H, D), np.uint16)), bits_dev(k), bits_dev(v),
                            o, 0.0883883)
    mean = bf16_to_f64(v).mean(axis=1)
    got = bf16_to_f64(host_bits(o))
    for a in range(A):
        assert np.max(np.abs(got[:, a] - mean)) < 2e-3


# ----------------------------------------------------------------------------- Euler

@pytest.mark.parametrize("N,C,frac", [(1000, 64, 0.4), (257, 3, 0.5), (32760, 64, 0.5),
                                      (10, 16, 0.0), (10, 16, 1.0)])
def test_euler(hs, N, C, frac):
    r = np.random.default_rng(N + C)
    x = r.standard_normal((N, C)).astype(np.float32)
    vh = r.standard_normal((N, C)).astype(np.float32)
    na = int(round(frac * N))
    idx = np.sort(r.choice(N, na, replace=False)).astype(np.int32)
    pos = np.full(N, -1, np.int32)
    pos[idx] = np.arange(na, dtype=np.int32)
    vf = r.standard_normal((max(na, 1), C)).astype(np.float32)
    sig = oracle.sigma_schedule(40)
    xd, vd = dev(x), dev(vh)
    hs.hsa_euler_step(xd, vd, dev(vf), dev(pos), na, float(sig[7]), float(sig[8]))
    xw, vw = oracle.euler_step(x, vh, vf[:na], idx, sig[7], sig[8])
    assert np.array_equal(host(vd), vw)
    assert np.array_equal(host(xd).view(np.uint32), xw.view(np.uint32))


# ----------------------------------------------------------------------------- whole loop

def run_loop_both(cfg, hs, layers=None, reselect=False):
    from sparse_attention_l1_amd.sampler import HsaSampler
    L = cfg.layers if layers is None else layers
    model = SyntheticModel(cfg, hs)
    scale = float(np.float32(1.0 / np.sqrt(cfg.head_dim)))
    rec = {}
    oracle.run_hsa(synth.latent0(cfg), model.vm.v_prev, model.vm, model.src.rows, model.src.prefill,
                   T=cfg.T, budgets=cfg.budgets, group_sizes=cfg.sizes, m=cfg.m, layers=L,
                   scale=scale, v_cur_for_m0=model.vm(0), record=lambda i, s: rec.__setitem__(i, s),
                   reselect=reselect)
    smp = HsaSampler(n_tokens=cfg.n_tokens, channels=cfg.channels, batch=cfg.batch, heads=cfg.heads,
                     head_dim=cfg.head_dim, layers=L, T=cfg.T, budgets=cfg.budgets,
                     group_sizes=cfg.sizes, m=cfg.m, softmax_scale=scale, reselect=reselect)
    smp.reset(dev(synth.latent0(cfg)), dev(model.vm.v_prev), model.prefill)
    if cfg.m == 0:
        smp.select(dev(model.vm.v_prev), dev(model.vm(0)))
    for i in range(cfg.T):
        outs = {}
        x_before = host(smp.x)
        smp.iteration(i, model, on_attention=lambda l, o: outs.__setitem__(l, host_bits(o)))
        torch.cuda.synchronize()
        want = rec[i]
        na = smp.n_active
        # the model's input rows gathered with the active set
        assert np.array_equal(host(smp.x_active)[:na].view(np.uint32),
                              x_before[want["active_idx"]].view(np.uint32)), f"iteration {i}"
        assert na == want["active_idx"].shape[0], f"iteration {i}"
        assert np.array_equal(host(smp.active_idx)[:na], want["active_idx"]), f"iteration {i}"
        assert np.array_equal(host(smp.active_pos), want["active_pos"]), f"iteration {i}"
        assert np.array_equal(host(smp.group_id), want["group_id"]), f"iteration {i}"
        for l in range(L):
            assert np.array_equal(host_bits(smp.k_cache[l]), want["k_caches"][l]), f"i {i} l {l}"
            assert np.array_equal(host_bits(smp.v_cache[l]), want["v_caches"][l]), f"i {i} l {l}"
            attn_close(outs[l], want["attn"][l], f"loop i{i} l{l}")
        assert np.array_equal(host(smp.v_hat), want["v_hat"]), f"iteration {i}"
        assert np.array_equal(host(smp.x).view(np.uint32), want["x"].view(np.uint32)), f"iteration {i}"


def test_tiny_full_loop(hs):
    run_loop_both(synth.tiny(), hs)


def test_small_loop_three_groups_two_layers_pair(hs):
    cfg = synth.Config("small pair", 77, 600, 8, 2, 2, 128, 2, 8, (8, 4, 2), (100, 200, 300), 2,
                       drift="student_t3")
    run_loop_both(cfg, hs)


def test_small_loop_no_window(hs):
    cfg = synth.Config("m0", 78, 300, 16, 1, 1, 64, 1, 4, (4, 2, 1), (50, 50, 200), 0)
    run_loop_both(cfg, hs)


def test_loop_reselect_at_every_all_active_iteration(hs):
    # groups recomputed at i = 1, 4, 8, 12, 16 and the closing window 18, 19 (periods 1, 2, 4;
    # m = 2)
    cfg = synth.Config("reselect", 79, 700, 16, 2, 2, 64, 2, 20, (20, 10, 5), (100, 200, 400), 2,
                       drift="student_t3")
    run_loop_both(cfg, hs, reselect=True)


def test_tiny_loop_reselect(hs):
    run_loop_both(synth.tiny(), hs, reselect=True)


def test_single_step_full_size(hs):
    """N = 32760, 12 x 128 heads, half the tokens active: the measured configuration, through
    the same calls the benchmark step makes (the active set fused with the latent-row gather,
    attention through the workspace entry point), with every output compared in full except
    attention (64 sampled query rows)."""
    cfg = synth.single_step()
    N, C, H, D, i = cfg.n_tokens, cfg.channels, cfg.heads, cfg.head_dim, cfg.iteration
    model = SyntheticModel(cfg, hs)
    vp, vc = model.vm.v_prev, model.vm(0)
    g_want, r_want = oracle.select_groups(vp, vc, cfg.sizes)
    g = torch.empty(N, dtype=torch.int32, device="cuda")
    ws = hs.workspace(N, cfg.n_groups)
    hs.hsa_select_groups(dev(vp), dev(vc), cfg.sizes, g, None, ws)
    idx = torch.empty(N, dtype=torch.int32, device="cuda")
    pos = torch.empty(N, dtype=torch.int32, device="cuda")
    x0 = synth.latent0(cfg)
    xd = dev(x0)
    x_act = torch.full((N, C), np.nan, dtype=torch.float32, device="cuda")
    na = hs.hsa_active_set_gather(g, cfg.budgets, cfg.sizes, cfg.T, cfg.m, i, idx, pos, xd,
                                  x_act, ws)
    idx_w, pos_w = oracle.active_set(g_want, cfg.budgets, cfg.T, cfg.m, i)
    assert na == 16380 == idx_w.shape[0]
    assert np.array_equal(host(g), g_want)
    assert np.array_equal(host(idx)[:na], idx_w) and np.array_equal(host(pos), pos_w)
    assert np.array_equal(host(x_act)[:na].view(np.uint32), x0[idx_w].view(np.uint32))
    assert np.isnan(host(x_act)[na:]).all()       # rows past |A| untouched

    pre = model.src.prefill(0)
    q, kn, vn = (model.src.rows(t, 0, i, na) for t in ("q", "k", "v"))
    kd, vd = bits_dev(pre), bits_dev(pre)
    hs.hsa_kv_update(kd, vd, bits_dev(kn), bits_dev(vn), idx, na)
    kc, vc_ = pre.copy(), pre.copy()
    oracle.kv_update(kc, vc_, kn, vn, idx_w)
    assert np.array_equal(host_bits(kd), kc) and np.array_equal(host_bits(vd), vc_)

    o = torch.empty((1, na, H, D), dtype=torch.int16, device="cuda")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    hs.hsa_attention_active_ws(bits_dev(q), kd, vd, o, scale,
                               hs.attention_workspace(na, N, 1, H, D))
    rows = synth.sample_rows(cfg.cfg_id, na, 64)
    want = oracle.attention_active(q[:, rows], kc, vc_, scale)
    attn_close(host_bits(o)[:, rows], want, "single step sampled rows")

    vhat0 = vp
    vhd = dev(vhat0)
    vfresh = model.velocity(i, idx, na)
    sig = oracle.sigma_schedule(cfg.T)
    hs.hsa_euler_step(xd, vhd, vfresh, pos, na, float(sig[i]), float(sig[i + 1]))
    xw, vw = oracle.euler_step(x0, vhat0, model.vm(i)[idx_w], idx_w, sig[i], sig[i + 1])
    assert np.array_equal(host(vhd), vw)
    assert np.array_equal(host(xd).view(np.uint32), xw.view(np.uint32))


def test_aggressive_pair_full_size_loop(hs):
    """B = 2 (a cond/uncond pair), N = 75600, 40 x 128 heads, T = 40, budgets {40, 10, 5} over
    10/30/60% of the tokens, heavy-tailed drift, m = 2, one layer: the whole 40-iteration loop
    through the C ABI.  Active sets, group ids, the latent and the velocity cache are compared
    in full at every iteration.  At iteration 37 (10% of the tokens active, so most cache rows
    are stale) sampled cache rows are compared with the replay rule (a row holds the K/V of the
    last iteration that had its token active, else the prefill) and attention with the oracle
    on sampled query rows, the oracle's caches rebuilt by that rule.  The sampler's attention
    splits the key range of the last round's query tiles at that iteration (2304 whole tiles,
    96 split in 5)."""
    cfg = synth.aggressive_pair()
    assert hs.hsastep_attention_plan(cfg.sizes[0], cfg.n_tokens, cfg.batch, cfg.heads,
                                     cfg.head_dim, 256, 1 << 40)[2] > 1
    _full_size_loop(hs, cfg, 37, "pair loop")


def test_full_schedule_full_size_loop(hs):
    """N = 32760, 12 x 128 heads, T = 40, four groups of 25% with budgets {40, 20, 10, 5},
    m = 4, one layer of the 30-layer stack: the whole 40-iteration loop through the C ABI, with
    the checks of the pair loop at iteration 33, where only G_1 is active (25%: 384 query
    tiles, so the last round's 128 tiles split their key range in two)."""
    cfg = synth.full_schedule()
    assert hs.hsastep_attention_plan(cfg.sizes[0], cfg.n_tokens, cfg.batch, cfg.heads,
                                     cfg.head_dim, 256, 1 << 40)[2] > 1
    _full_size_loop(hs, cfg, 33, "full schedule loop")


def _full_size_loop(hs, cfg, check_i, tag):
    from sparse_attention_l1_amd.sampler import HsaSampler
    N, H, D, T, B = cfg.n_tokens, cfg.heads, cfg.head_dim, cfg.T, cfg.batch
    model = SyntheticModel(cfg, hs)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    rec = {}
    oracle.run_hsa(synth.latent0(cfg), model.vm.v_prev, model.vm, model.src.rows,
                   model.src.prefill, T=T, budgets=cfg.budgets, group_sizes=cfg.sizes, m=cfg.m,
                   layers=0, scale=scale,
                   record=lambda i, s: rec.__setitem__(i, {k: s[k] for k in
                                                           ("active_idx", "group_id", "x", "v_hat")}))
    assert rec[check_i]["active_idx"].shape[0] == cfg.sizes[0]
    smp = HsaSampler(n_tokens=N, channels=cfg.channels, batch=B, heads=H, head_dim=D, layers=1,
                     T=T, budgets=cfg.budgets, group_sizes=cfg.sizes, m=cfg.m, softmax_scale=scale)
    smp.reset(dev(synth.latent0(cfg)), dev(model.vm.v_prev), model.prefill)
    qrows = synth.sample_rows(cfg.cfg_id, cfg.sizes[0], 24, tag=1)
    crow = synth.sample_rows(cfg.cfg_id, N, 256, tag=2)
    got = {}

    def observe(l, o):
        if smp_i[0] == check_i:
            got["attn"] = host_bits(o[:, torch.from_numpy(qrows).cuda()])
            got["k"] = host_bits(smp.k_cache[0][:, torch.from_numpy(crow).cuda()])
            got["v"] = host_bits(smp.v_cache[0][:, torch.from_numpy(crow).cuda()])

    smp_i = [0]
    for i in range(T):
        smp_i[0] = i
        smp.iteration(i, model, on_attention=observe)
        torch.cuda.synchronize()
        want = rec[i]
        na = smp.n_active
        print(f"[{tag}] iteration {i}: {na} active", flush=True)
        assert na == want["active_idx"].shape[0], f"iteration {i}"
        assert np.array_equal(host(smp.active_idx)[:na], want["active_idx"]), f"iteration {i}"
        assert np.array_equal(host(smp.group_id), want["group_id"]), f"iteration {i}"
        assert np.array_equal(host(smp.v_hat), want["v_hat"]), f"iteration {i}"
        assert np.array_equal(host(smp.x).view(np.uint32), want["x"].view(np.uint32)), f"iteration {i}"

    # replay rule for layer 0 after the scatter of iteration check_i
    last = np.full(N, -1, np.int64)
    pos = np.zeros(N, np.int64)
    for j in range(check_i + 1):
        idx = rec[j]["active_idx"]
        last[idx] = j
        pos[idx] = np.arange(idx.shape[0])
    caches = {}
    for t in ("k", "v"):
        c = model.src.prefill(0)
        for j in np.unique(last[last >= 0]):
            toks = np.flatnonzero(last == j)
            need = rec[j]["active_idx"].shape[0] * H * D
            for b in range(B):
                win = model.src.pools[t].window(need, b, 0, j).reshape(-1, H, D)
                c[b, toks] = win[pos[toks]]
        caches[t] = c
        assert np.array_equal(got[t], c[:, crow]), f"cache {t} rows at iteration {check_i}"
    na = rec[check_i]["active_idx"].shape[0]
    q = model.src.rows("q", 0, check_i, na)[:, qrows]
    want = oracle.attention_active(q, caches["k"], caches["v"], scale)
    attn_close(got["attn"], want, f"{tag} i{check_i} sampled rows")


# ----------------------------------------------------------------------------- active set + gather

@pytest.mark.parametrize("N,row_words,budgets,sizes,T,m,it", [
    (32760, 64, (40, 20), (16380, 16380), 40, 4, 5),          # fp32 latent rows, vector path
    (1000, 3, (8, 4), (300, 700), 8, 1, 3),                   # 12-byte rows, word path
    (5000, 65, (12, 6, 3), (1000, 1500, 2500), 12, 0, 4),    # 260-byte rows
    (3000, 16, (8, 4), (0, 3000), 8, 1, 3),                   # no active token at all
])
def test_active_set_gather(hs, N, row_words, budgets, sizes, T, m, it):
    rng = np.random.default_rng(N + row_words)
    g_host = rng.permutation(np.repeat(np.arange(len(sizes)), sizes)).astype(np.int32)
    rows = rng.standard_normal((N, row_words)).astype(np.float32)
    g = dev(g_host)
    idx = torch.full((N,), -9, dtype=torch.int32, device="cuda")
    pos = torch.empty(N, dtype=torch.int32, device="cuda")
    out = torch.full((N + 1, row_words), 7.0, dtype=torch.float32, device="cuda")
    na = hs.hsa_active_set_gather(g, budgets, sizes, T, m, it, idx, pos, dev(rows), out,
                                  hs.workspace(N, len(budgets)))
    torch.cuda.synchronize()
    want_idx, want_pos = oracle.active_set(g_host, budgets, T, m, it)
    assert na == want_idx.shape[0]
    assert np.array_equal(host(idx)[:na], want_idx) and np.all(host(idx)[na:] == -9)
    assert np.array_equal(host(pos), want_pos)
    got = host(out)
    assert np.array_equal(got[:na].view(np.uint32), rows[want_idx].view(np.uint32))
    assert np.all(got[na:] == 7.0)                 # nothing written past |A_i|
