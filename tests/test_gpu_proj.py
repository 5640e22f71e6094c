"""GPU parity of hsa_qkv_project (the fused QKV projection of the active tokens, with the
KV-cache write as its epilogue) against the oracle, through the C ABI.

Bars: cache rows whose slot is not active are bit-identical to before the call; q_out and
the active cache rows are within 2^-8 |y| + 2^-12 S of the float64 product y, where
S = sum_k |x_k w_k| bounds the fp32 accumulation error (bf16 products are exact in fp32)
and 2^-8 |y| covers the bf16 rounding of the output (half an ulp is at most 2^-9 |y|).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_l1_amd import synth
from tests.gpu_helpers import bits_dev, dev, host_bits, bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


def bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def close(got_bits, want, bound, label):
    got = bf16_to_f64(got_bits)
    err = np.abs(got - want)
    lim = 2.0 ** -8 * np.abs(want) + 2.0 ** -12 * bound
    print(f"[{label}] max err {err.max():.3e}, max err / bound {np.max(err / lim):.3f}", flush=True)
    assert np.all(err <= lim), label


def offset_copy(t):
    """The same values at a device address 2 bytes past an 8-byte boundary."""
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    out = flat[1:].view(t.shape)
    out.copy_(t)
    return out


def run_case(hs, B, A, N, H, D, Dm, with_bias, seed, bad_slot=False, sample=None, misalign=False):
    r = np.random.default_rng(seed)
    HD = H * D
    x = bits(r.standard_normal((B, A, Dm)) * 0.5)
    w = bits(r.standard_normal((3 * HD, Dm)) / np.sqrt(Dm))
    bias = bits(r.standard_normal(3 * HD) * 0.1) if with_bias else None
    idx = np.sort(r.choice(N, A, replace=False)).astype(np.int32)
    if bad_slot:
        idx[-1] = N + 5          # outside [0, N): that row's K/V are skipped
    kc0 = bits(r.standard_normal((B, N, H, D)))
    vc0 = bits(r.standard_normal((B, N, H, D)))
    kd, vd = bits_dev(kc0), bits_dev(vc0)
    q = torch.full((B, A, H, D), 0x7F7F, dtype=torch.int16, device="cuda")
    if misalign:
        kd, vd, q = offset_copy(kd), offset_copy(vd), offset_copy(q)
        assert q.data_ptr() % 8 == 2
    hs.hsa_qkv_project(bits_dev(x), bits_dev(w), None if bias is None else bits_dev(bias), q, kd,
                       vd, dev(idx), A)
    torch.cuda.synchronize()
    rows = np.arange(A) if sample is None else sample
    qw, kw, vw = oracle.qkv_project(x[:, rows], w, bias, H, D)
    ax = np.abs(oracle.bf16_bits_to_f64(x[:, rows]))
    aw = np.abs(oracle.bf16_bits_to_f64(w))
    S = (ax @ aw.T).reshape(B, rows.size, 3, H, D)
    close(host_bits(q)[:, rows], qw, S[:, :, 0], f"q B{B} A{A} Dm{Dm}")
    valid = (idx >= 0) & (idx < N)
    for name, got_dev, c0, want, p in (("k", kd, kc0, kw, 1), ("v", vd, vc0, vw, 2)):
        got = host_bits(got_dev)
        untouched = np.ones(N, bool)
        untouched[idx[valid]] = False
        assert np.array_equal(got[:, untouched], c0[:, untouched]), f"{name}: stale rows changed"
        sel = valid[rows]
        close(got[:, idx[rows[sel]]], want[:, sel], S[:, sel, p], f"{name} cache B{B} A{A}")


@pytest.mark.parametrize("B,A,N,H,D,Dm,with_bias", [
    (1, 1, 5, 2, 64, 64, False),          # one row
    (2, 300, 500, 3, 64, 128, True),      # ragged row and column tiles, batch 2, bias
    (1, 1000, 2000, 12, 128, 1536, False),
    (1, 257, 300, 1, 64, 320, True),      # 3*H*D = 192 < one column tile
    (1, 513, 1000, 2, 64, 192, False),    # three stages of the reduction (odd count)
    (1, 300, 700, 3, 30, 128, True),      # H*D = 90: columns of a 4-group straddle q/k/v
    (2, 100, 400, 1, 6, 64, True),        # H*D = 6, one stage
])
def test_qkv_project(hs, B, A, N, H, D, Dm, with_bias):
    run_case(hs, B, A, N, H, D, Dm, with_bias, seed=A + N + Dm)


def test_qkv_project_unaligned_destinations(hs):
    """q_out and the caches 2 bytes off an 8-byte boundary: per-value stores."""
    run_case(hs, 2, 300, 500, 3, 64, 128, True, seed=17, misalign=True)


def test_qkv_project_skips_invalid_slot(hs):
    run_case(hs, 1, 64, 100, 2, 64, 64, True, seed=9, bad_slot=True)


def test_qkv_project_unaligned_many_tiles(hs):
    """More tiles than workgroups (each walks several) on the per-value store path."""
    rows = synth.sample_rows(1, 9000, 48, tag=5)
    run_case(hs, 1, 9000, 12000, 8, 96, 1024, True, seed=21, sample=rows, misalign=True)


@pytest.mark.parametrize("B,A,N,H,D,Dm,with_bias", [
    (2, 300, 500, 3, 64, 4096, True),     # 64 stages: the smallest rotated reduction, 9 tiles
    (1, 700, 1000, 8, 64, 4160, False),   # 65 stages (odd), ragged tiles, 18 rotations
])
def test_qkv_project_rotated_start(hs, B, A, N, H, D, Dm, with_bias):
    """Reductions of 64 stages or more start at a per-tile stage and wrap around."""
    run_case(hs, B, A, N, H, D, Dm, with_bias, seed=A + Dm)


def test_qkv_project_rotated_many_tiles_unaligned(hs):
    """More tiles than rotation positions (96), on the per-value store path."""
    rows = synth.sample_rows(1, 2000, 48, tag=7)
    run_case(hs, 1, 2000, 3000, 16, 64, 4096, True, seed=23, sample=rows, misalign=True)


def test_qkv_project_model_dim_5120(hs):
    """The pair's projection shape at model dim 5120 (80 stages, 3540 tiles over 40 x 128
    heads, batch 2, bias) on a smaller cache: 64 sampled rows against the oracle, every
    stale cache row bit for bit."""
    rows = synth.sample_rows(2, 7560, 32, tag=9)
    run_case(hs, 2, 7560, 8000, 40, 128, 5120, True, seed=29, sample=rows)


def test_qkv_project_full_size_single_step(hs):
    """16380 active rows of a 32760-token cache, 12 x 128 heads, model dim 1536: every stale
    row checked bit for bit, 64 sampled rows against the oracle."""
    rows = synth.sample_rows(1, 16380, 64, tag=3)
    run_case(hs, 1, 16380, 32760, 12, 128, 1536, True, seed=11, sample=rows)

