"""One HSA iteration captured in a HIP graph and replayed.

Every entry point launches kernels on the caller's stream only: no allocation, no memset, no
host synchronisation, and the active count comes from the host-side schedule.  So one whole
iteration (selection, active set, gather, cache scatter or fused projection, attention,
cached Euler update) can be captured once and replayed, also with the fused active-set
gather, the split attention and its merge kernel, and the allocation-free active set (whose
scratch address is looked up by the eager call before the capture).  Each replay starts from the same
state, with eager work and synchronisations between replays, and must reproduce the eager
iteration bit for bit.
"""
import numpy as np
import pytest
import torch

from sparse_attention_l1_amd import synth
from tests.gpu_helpers import bits_dev, dev

pytestmark = pytest.mark.gpu

N, C, H, D, DM = 4000, 64, 2, 128, 256
SIZES, BUDGETS, T, M, ITER = (1500, 2500), (8, 4), 8, 1, 3


@pytest.fixture(scope="module")
def hs():
    from sparse_attention_l1_amd import hsastep
    return hsastep


def _state(hs):
    r = np.random.default_rng(11)
    vp = r.standard_normal((N, C)).astype(np.float32)
    lam = r.lognormal(0, 1, N).astype(np.float32)
    vc = (vp + lam[:, None] * r.standard_normal((N, C)).astype(np.float32)).astype(np.float32)
    na = hs.hsastep_n_active(N, BUDGETS, SIZES, T, M, ITER)
    bf = lambda *shape: bits_dev(synth.f32_to_bf16_bits(r.standard_normal(shape).astype(np.float32)))
    st = {
        "v_prev": dev(vp), "v_cur": dev(vc),
        "v_model": dev(r.standard_normal((N, C)).astype(np.float32)),
        "x": dev(r.standard_normal((N, C)).astype(np.float32)),
        "v_hat": dev(vp.copy()),
        "k_cache": bf(1, N, H, D), "v_cache": bf(1, N, H, D),
        "q": bf(1, na, H, D), "k_new": bf(1, na, H, D), "v_new": bf(1, na, H, D),
        "x_model": bf(1, na, DM), "w": bits_dev(synth.f32_to_bf16_bits(
            (r.standard_normal((3 * H * D, DM)) / np.sqrt(DM)).astype(np.float32))),
        "bias": bf(3 * H * D),
        "group_id": torch.empty(N, dtype=torch.int32, device="cuda"),
        "active_idx": torch.empty(N, dtype=torch.int32, device="cuda"),
        "active_pos": torch.empty(N, dtype=torch.int32, device="cuda"),
        "x_act": torch.zeros((N, C), dtype=torch.float32, device="cuda"),
        "v_fresh": torch.empty((na, C), dtype=torch.float32, device="cuda"),
        "q_proj": torch.empty((1, na, H, D), dtype=torch.int16, device="cuda"),
        "out": torch.empty((1, na, H, D), dtype=torch.int16, device="cuda"),
        "ws": hs.workspace(N, len(SIZES)),
        "attn_ws": hs.attention_workspace(na, N, 1, H, D),
    }
    return st, na


def _iteration(hs, st, variant):
    """variant: "plain" (separate calls), "fused" (projection with the cache write),
    "ws" (active set fused with the latent gather; attention with a workspace, whose tiles are
    all split here: 2 query tiles on a 256-CU chip), "noalloc" (the allocation-free active
    set)."""
    fused = variant == "fused"
    hs.hsa_select_groups(st["v_prev"], st["v_cur"], SIZES, st["group_id"], None, st["ws"])
    if variant == "ws":
        na = hs.hsa_active_set_gather(st["group_id"], BUDGETS, SIZES, T, M, ITER,
                                      st["active_idx"], st["active_pos"], st["x"], st["x_act"],
                                      st["ws"])
    else:
        if variant == "noalloc":
            na = hs.hsa_active_set_noalloc(st["group_id"], BUDGETS, SIZES, T, M, ITER,
                                           st["active_idx"], st["active_pos"])
        else:
            na = hs.hsa_active_set(st["group_id"], BUDGETS, SIZES, T, M, ITER, st["active_idx"],
                                   st["active_pos"], st["ws"])
        hs.hsastep_gather_rows(st["x_act"], st["x"], st["active_idx"], na)
    hs.hsastep_gather_rows(st["v_fresh"], st["v_model"], st["active_idx"], na)
    if fused:
        hs.hsa_qkv_project(st["x_model"], st["w"], st["bias"], st["q_proj"], st["k_cache"],
                           st["v_cache"], st["active_idx"], na)
        q = st["q_proj"]
    else:
        hs.hsa_kv_update(st["k_cache"], st["v_cache"], st["k_new"], st["v_new"],
                         st["active_idx"], na)
        q = st["q"]
    if variant == "ws":
        hs.hsa_attention_active_ws(q, st["k_cache"], st["v_cache"], st["out"], 1.0 / np.sqrt(D),
                                   st["attn_ws"])
    else:
        hs.hsa_attention_active(q, st["k_cache"], st["v_cache"], st["out"], 1.0 / np.sqrt(D))
    hs.hsa_euler_step(st["x"], st["v_hat"], st["v_fresh"], st["active_pos"], na, 0.625, 0.5)


OUTPUTS = ("group_id", "active_idx", "active_pos", "x_act", "v_fresh", "q_proj", "k_cache",
           "v_cache", "out", "x", "v_hat")


@pytest.mark.parametrize("fused", ["plain", "fused", "ws", "noalloc"])
def test_iteration_graph_replays_match_eager(hs, fused):
    st, na = _state(hs)
    assert 0 < na < N
    st["q_proj"].zero_()
    st["out"].zero_()
    initial = {k: t.clone() for k, t in st.items()}

    def reset():
        for k, t in initial.items():
            st[k].copy_(t)

    _iteration(hs, st, fused)
    torch.cuda.synchronize()
    eager = {k: st[k].clone() for k in OUTPUTS}
    assert not torch.equal(eager["x"], initial["x"])

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _iteration(hs, st, fused)
    torch.cuda.synchronize()

    side = torch.empty_like(st["out"])
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in OUTPUTS:
            assert torch.equal(st[k], eager[k]), f"replay {rep}: {k} differs from the eager run"
        # eager work between replays, on the same buffers the graph reads
        hs.hsa_attention_active(st["q"], st["k_cache"], st["v_cache"], side, 0.5)
        torch.cuda.synchronize()


def test_iteration_on_a_side_stream_matches(hs):
    """Every launch goes to the caller's stream: the iteration issued on a side stream (default
    priority) gives the same bits as on the current stream."""
    st, na = _state(hs)
    st["q_proj"].zero_()
    st["out"].zero_()
    initial = {k: t.clone() for k, t in st.items()}
    _iteration(hs, st, "plain")
    torch.cuda.synchronize()
    want = {k: st[k].clone() for k in OUTPUTS}
    for k, t in initial.items():
        st[k].copy_(t)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _iteration(hs, st, "plain")
    side.synchronize()
    for k in OUTPUTS:
        assert torch.equal(st[k], want[k]), f"{k} differs on the side stream"
