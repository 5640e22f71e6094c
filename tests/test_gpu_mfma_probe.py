"""The MFMA rate probe does the work it is timed for.

Each wavefront keeps 8 accumulators; accumulator k receives A_k . B_((k+j) mod 8) for
j = 0..7 in every round, where A_i and B_i are 32x16 and 16x32 bf16 tiles read from the
operand buffer (lane l holds row or column l mod 32, k elements 8*(l div 32) .. +8).  The
sum of every element of every accumulator over a wavefront's 64 lanes is therefore
rounds * sum_k sum_j colsum(A_k) . rowsum(B_j), which does not depend on how the result
tile is spread over the lanes.  The probe writes per-lane sums, so the sum over each
wavefront's lanes must match that on every wavefront of every workgroup.
"""
import numpy as np
import pytest
import torch

from sparse_attention_l1_amd import synth

pytestmark = pytest.mark.gpu


def _expected_wave_sum(bits: np.ndarray, rounds: int) -> float:
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(1024, 8)
    # operand group i (A for i < 8, B for i >= 8) is lanes 64 i .. 64 i + 63; k = 8 (l div 32) + e
    groups = vals.reshape(16, 2, 32, 8)                 # [group, lane div 32, lane mod 32, e]
    ksum = groups.sum(axis=2).reshape(16, 16)           # [group, k]: A colsums / B rowsums
    a, b = ksum[:8], ksum[8:]
    return rounds * float((a.sum(axis=0) * b.sum(axis=0)).sum())


@pytest.mark.parametrize("rounds,workgroups", [(1, 3), (5, 300)])
def test_probe_wave_sums(rounds, workgroups):
    from sparse_attention_l1_amd import hsastep as hs
    r = np.random.default_rng(rounds)
    vals = (r.uniform(0.25, 2.0, hs.MFMA_PROBE_OPERANDS)
            * r.choice([-1.0, 1.0], hs.MFMA_PROBE_OPERANDS)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    ops = torch.from_numpy(bits.view(np.int16)).cuda()
    sink = torch.full((workgroups * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = hs.hsastep_mfma_probe(ops, sink, rounds, workgroups)
    torch.cuda.synchronize()
    assert flops == workgroups * 4 * 64 * rounds * 32768
    got = sink.cpu().numpy().astype(np.float64).reshape(workgroups * 4, 64).sum(axis=1)
    want = _expected_wave_sum(bits, rounds)
    scale = rounds * 8 * 8 * 32 * 32 * 16 * 4.0    # bound on the sum of |products|
    assert np.abs(got - want).max() <= 1e-6 * scale, (got[:4], want)


def test_probe_rejects_bad_arguments():
    from sparse_attention_l1_amd import hsastep as hs
    ops = torch.zeros(hs.MFMA_PROBE_OPERANDS, dtype=torch.int16, device="cuda")
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    with pytest.raises(hs.HsaStepError):
        hs.hsastep_mfma_probe(ops, sink, 0, 1)
    with pytest.raises(ValueError):
        hs.hsastep_mfma_probe(ops, sink, 1, 2)
