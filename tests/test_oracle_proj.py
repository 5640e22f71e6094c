"""Pins for the oracle's QKV projection of the active tokens.

"Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor Efficiënte
Videogeneratie" §2.2 items 1-2: only the active tokens go through the model's
projections, and their fresh K/V rows are what the cache takes.  The oracle is a plain
float64 product; it is pinned to a library routine (torch's linear in float64 on the
CPU), to hand values, and to the split of the stacked weight into its three parts.
"""
import numpy as np
import torch

import oracle
from sparse_attention_l1_amd import synth


def bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_matches_library_linear():
    r = np.random.default_rng(3)
    B, A, Dm, H, D = 2, 7, 64, 3, 8
    x, w, b = bits(r.standard_normal((B, A, Dm))), bits(r.standard_normal((3 * H * D, Dm))), \
        bits(r.standard_normal(3 * H * D))
    q, k, v = oracle.qkv_project(x, w, b, H, D)
    f = lambda t: torch.from_numpy(oracle.bf16_bits_to_f64(t))
    y = torch.nn.functional.linear(f(x), f(w), f(b)).numpy()
    got = np.concatenate([t.reshape(B, A, -1) for t in (q, k, v)], -1)
    np.testing.assert_allclose(got, y, rtol=1e-13, atol=1e-12)


def test_hand_values():
    # Dm = 2, H = 1, D = 1: rows of W pick / combine the two input features
    x = bits([[[1.0, 2.0], [3.0, -1.0]]])                 # B = 1, |A| = 2
    w = bits([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])        # q = x0, k = x1, v = x0 + x1
    q, k, v = oracle.qkv_project(x, w, bits([0.0, 0.5, -1.0]), 1, 1)
    assert q.ravel().tolist() == [1.0, 3.0]
    assert k.ravel().tolist() == [2.5, -0.5]
    assert v.ravel().tolist() == [2.0, 1.0]


def test_stacked_weight_splits_into_three_products():
    r = np.random.default_rng(4)
    B, A, Dm, H, D = 1, 5, 32, 2, 4
    x = bits(r.standard_normal((B, A, Dm)))
    w = bits(r.standard_normal((3 * H * D, Dm)))
    q, k, v = oracle.qkv_project(x, w, None, H, D)
    xf = oracle.bf16_bits_to_f64(x)
    for p, out in enumerate((q, k, v)):
        wp = oracle.bf16_bits_to_f64(w[p * H * D:(p + 1) * H * D])
        np.testing.assert_allclose(out.reshape(B, A, H * D), xf @ wp.T, rtol=1e-13, atol=1e-12)
