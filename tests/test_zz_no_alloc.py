"""hsa_active_set_noalloc (the active set without a workspace, for callers that cannot
allocate) against hsa_active_set, through the C ABI.

Two calls in a row on the same device, the second with fewer tokens, so the second runs on
the counts the first left in the library's scratch array; each output must equal the
workspace entry point's bit for bit (the index list and the inverse map), and |A_i| must
match.  A call above the limit is rejected before anything is enqueued.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


def _groups(n, sizes, seed):
    rng = np.random.default_rng(seed)
    g = rng.permutation(np.repeat(np.arange(len(sizes)), sizes)).astype(np.int32)
    return torch.from_numpy(g).cuda()


def _both(hs, g, budgets, sizes, T, m, i):
    n = g.shape[0]
    idx_a = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pos_a = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    idx_b = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pos_b = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    na_a = hs.hsa_active_set(g, budgets, sizes, T, m, i, idx_a, pos_a,
                             hs.workspace(n, len(budgets)))
    na_b = hs.hsa_active_set_noalloc(g, budgets, sizes, T, m, i, idx_b, pos_b)
    torch.cuda.synchronize()
    return (na_a, idx_a.cpu().numpy(), pos_a.cpu().numpy()), \
           (na_b, idx_b.cpu().numpy(), pos_b.cpu().numpy())


@pytest.mark.parametrize("first,second", [
    # (n_tokens, budgets, sizes, T, m, iteration) of the two calls; the second is smaller
    ((75600, (40, 10, 5), (7560, 22680, 45360), 40, 2, 8),
     (32760, (40, 20, 10, 5), (8190, 8190, 8190, 8190), 40, 4, 6)),
    ((32760, (40, 20), (16380, 16380), 40, 4, 5),
     (1000, (8, 4), (300, 700), 8, 1, 3)),
])
def test_noalloc_matches_workspace_entry_point(hs, first, second):
    for k, (n, budgets, sizes, T, m, i) in enumerate((first, second)):
        print(f"[no-alloc] call {k}: N={n} budgets={budgets} iteration={i}", flush=True)
        g = _groups(n, sizes, n + i)
        (na_a, idx_a, pos_a), (na_b, idx_b, pos_b) = _both(hs, g, budgets, sizes, T, m, i)
        assert na_a == na_b == hs.hsastep_n_active(n, budgets, sizes, T, m, i)
        assert np.array_equal(idx_a[:na_a], idx_b[:na_b])
        assert np.all(idx_b[na_b:] == -7)          # nothing written past |A_i|
        assert np.array_equal(pos_a, pos_b)


def test_noalloc_rejects_more_tokens_than_its_scratch(hs):
    n = hs.NOALLOC_MAX_TOKENS + 1
    g = torch.zeros(n, dtype=torch.int32, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int32, device="cuda")
    with pytest.raises(hs.HsaStepError) as e:
        hs.hsa_active_set_noalloc(g, (8,), (n,), 8, 1, 0, idx, pos)
    assert e.value.code == hs.ERR_UNSUPPORTED
