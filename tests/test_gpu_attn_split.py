"""GPU parity of the attention path with a workspace (hsa_attention_active_ws): the query
tiles of a last round that would leave compute units idle are split into key ranges whose
partial results a second kernel merges ([HSA-nl] §2.2 item 4: the cost is O(|A_i| * N), so
iterations with few active tokens launch few tiles).

Each case is checked element by element against the float64 oracle at the same 2e-2 bar as
the unsplit path, and against the unsplit kernel itself.  The plan each case gets comes from the library's planner
(hsastep_attention_plan, printed); the cases cover every tile split (launches smaller than
the chip), whole and split tiles mixed, a split count that is not a power of two, ragged key
counts, B = 2, a workspace too small for the best plan, and no workspace (then the bits equal
hsa_attention_active's).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_l1_amd import synth
from tests.gpu_helpers import attn_close, bits_dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


def _inputs(B, A, N, H, seed, qs=1.0):
    r = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits((r.standard_normal((B, A, H, 128)) * qs).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, 128)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, N, H, 128)).astype(np.float32))
    return q, k, v


# B, |A|, N, H, q scale, rows compared with the oracle (None = all)
CASES = [
    (2, 300, 3000, 3, 1.0, None),      # 12 tiles: every tile split, 8 key ranges
    (2, 300, 3003, 3, 8.0, None),      # ragged N, peaky
    (1, 70, 32 * 40 - 5, 2, 1.0, None),  # ragged N over 2 tiles
    (1, 513, 700, 1, 1.0, None),       # N = 700: two key ranges at most
    (2, 1100, 20000, 40, 1.0, 24),     # 400 tiles: 256 whole, 144 split in 3
    (1, 16380, 32760, 12, 1.0, 24),    # 768 tiles = 3 full rounds: nothing split
]


@pytest.mark.parametrize("B,A,N,H,qs,rows", CASES)
def test_split_attention_matches_oracle(hs, B, A, N, H, qs, rows):
    q, k, v = _inputs(B, A, N, H, A + N, qs)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    qd, kd, vd = bits_dev(q), bits_dev(k), bits_dev(v)
    ws = hs.attention_workspace(A, N, B, H, 128)
    o = torch.full((B, A, H, 128), 0x7F7F, dtype=torch.int16, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = hs.hsastep_attention_plan(A, N, B, H, 128, cus, ws.numel())
    print(f"[split] B{B} A{A} N{N} H{H}: plan {plan} on {cus} CUs", flush=True)
    hs.hsa_attention_active_ws(qd, kd, vd, o, scale, ws)
    o_plain = torch.empty_like(o)
    hs.hsa_attention_active(qd, kd, vd, o_plain, scale)
    torch.cuda.synchronize()
    sel = np.arange(A) if rows is None else synth.sample_rows(99, A, rows)
    want = oracle.attention_active(q[:, sel], k, v, scale)
    got = host_bits(o)
    attn_close(got[:, sel], want, f"split B{B} A{A} N{N} H{H} x{qs}")
    # against the unsplit kernel: each key range has its own reference max, so its P values
    # round differently; both are within the oracle's bar, and so is their difference
    diff = float(np.max(np.abs(synth_bf16_to_f64(got) - synth_bf16_to_f64(host_bits(o_plain)))))
    print(f"[split] max |split - unsplit| {diff:.3e}", flush=True)
    assert diff <= 2e-2


@pytest.mark.parametrize("A", [75600, 37800, 18900, 9450], ids=["f1", "f1/2", "f1/4", "f1/8"])
def test_split_attention_sweep_shape(hs, A):
    """The large-head sweep's shapes (B = 1, |A| = f N of N = 75600 tokens, 40 x 128 heads;
    f = 1 is the largest launch of the workloads, 11840 tiles).  At f = 1/4, 2960 tiles: the
    last round's 144 are split in 3 key ranges.  Inputs are seeded N(0,1) values drawn on the
    device (as the benchmark's sweep draws them); 16 sampled query rows are compared with the
    oracle, and every row with the unsplit kernel."""
    B, N, H = 1, 75600, 40
    g = torch.Generator(device="cuda").manual_seed(20260512)
    draw = lambda *shape: torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    qd, kd, vd = draw(B, A, H, 128), draw(B, N, H, 128), draw(B, N, H, 128)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    ws = hs.attention_workspace(A, N, B, H, 128)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = hs.hsastep_attention_plan(A, N, B, H, 128, cus, ws.numel())
    print(f"[split] sweep shape A{A}: plan {plan} on {cus} CUs", flush=True)
    o = torch.full((B, A, H, 128), 0x7F7F, dtype=torch.int16, device="cuda")
    o_plain = torch.empty_like(o)
    hs.hsa_attention_active_ws(qd, kd, vd, o, scale, ws)
    hs.hsa_attention_active(qd, kd, vd, o_plain, scale)
    torch.cuda.synchronize()
    sel = synth.sample_rows(98, A, 16)
    bits = lambda t: t.cpu().numpy().view(np.uint16)
    want = oracle.attention_active(bits(qd)[:, sel], bits(kd), bits(vd), scale)
    got = host_bits(o)
    attn_close(got[:, sel], want, f"split sweep shape A{A}")
    # each output averages 75600 values, so |O| is far below the absolute bar: also hold the
    # error to 2^-6 of max|O| (the output's own rounding is up to 2^-9 of it)
    rel = float(np.max(np.abs(synth_bf16_to_f64(got[:, sel]) - want)))
    assert rel <= 2.0 ** -6 * float(np.max(np.abs(want)))
    diff = float(np.max(np.abs(synth_bf16_to_f64(got) - synth_bf16_to_f64(host_bits(o_plain)))))
    print(f"[split] sweep shape: max |split - unsplit| {diff:.3e}", flush=True)
    assert diff <= 2e-2


def synth_bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_small_workspace_and_none(hs):
    B, A, N, H = 2, 300, 3000, 3
    q, k, v = _inputs(B, A, N, H, 7)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    qd, kd, vd = bits_dev(q), bits_dev(k), bits_dev(v)
    want = oracle.attention_active(q, k, v, scale)
    piece = hs.hsastep_attention_workspace_bytes(A, N, B, H, 128) // min(12 * 8, 512)
    for nbytes in (piece * 12 * 2, piece * 12 * 2 + piece - 16, 16):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o = torch.empty((B, A, H, 128), dtype=torch.int16, device="cuda")
        hs.hsa_attention_active_ws(qd, kd, vd, o, scale, ws)
        torch.cuda.synchronize()
        attn_close(host_bits(o), want, f"split workspace {nbytes} bytes")
    o_none = torch.empty((B, A, H, 128), dtype=torch.int16, device="cuda")
    o_plain = torch.empty_like(o_none)
    hs.hsa_attention_active_ws(qd, kd, vd, o_none, scale, None)
    hs.hsa_attention_active(qd, kd, vd, o_plain, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_none, o_plain)


def test_split_is_deterministic(hs):
    B, A, N, H = 2, 300, 3000, 3
    q, k, v = _inputs(B, A, N, H, 8)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    qd, kd, vd = bits_dev(q), bits_dev(k), bits_dev(v)
    ws = hs.attention_workspace(A, N, B, H, 128)
    o1 = torch.empty((B, A, H, 128), dtype=torch.int16, device="cuda")
    o2 = torch.empty_like(o1)
    hs.hsa_attention_active_ws(qd, kd, vd, o1, scale, ws)
    hs.hsa_attention_active_ws(qd, kd, vd, o2, scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
