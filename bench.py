#!/usr/bin/env python3
"""Benchmark of one HSA denoise iteration on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-loop]
                    [--no-streaming] [--no-mfma-ceiling] [--pair] [--sweep] [--split] [--proj]

A step is one pass of the whole path over the single-step workload (N = 32760
tokens on a 21x30x52 latent grid, 12 heads x 128, 64 latent channels, half of
the tokens active): token selection by L1 relative velocity change, the active
set with the gather of the active latent rows, the KV-cache scatter, active-query
attention against all N cached rows, and the cached Euler update.  Inputs are
seeded synthetic data already resident in HBM.  Prints one JSON line.

value = attention FLOPs of the iteration (4 * |A| * N * H * D) / wall time of the
whole iteration, in TFLOP/s; ms_per_step is that wall time.  The roofline entry
is the attention kernel alone, timed with HIP events around each launch; mfma_ceiling
is the sustained rate of the same MFMA instruction with nothing else in the loop, and
attention's fraction of it.
The full 40-iteration, 30-layer schedule (T=40, budgets {40,20,10,5}, m=4) is also run
once and its mean ms per iteration reported (the metric's second half), as are the
HBM-bound kernels one by one with their fraction of 8 TB/s and a plain-copy ceiling at the
same sizes; --pair does the same for
the aggressive cond/uncond pair (B=2, N=75600, 40x128 heads, 40 layers, T=40, budgets
{40,10,5} over 10/30/60% of the tokens, m=2).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
ATTN_PMC_SUMMARY = os.path.join(ROOT, "profiles", "attention_single_step_pmc.txt")
# sources of the attention kernels: the counters summary is valid only for this exact code
# (the code of the two HIP files and the two key loops the generator emits; not comments)
ATTN_SRCS = [os.path.join(ROOT, "sparse_attention_l1_amd", "csrc", f)
             for f in ("attn.hip", "attn_pipe.hip")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10,
                   help="untimed steps first: the GPU clock ramps up over the first ~10 launches")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-loop", action="store_true",
                   help="skip the full 40-iteration, 30-layer schedule (run by default)")
    p.add_argument("--no-streaming", action="store_true",
                   help="skip the per-kernel HBM figures and the copy ceiling (run by default)")
    p.add_argument("--no-mfma-ceiling", action="store_true",
                   help="skip the sustained MFMA rate probe (run by default, ~0.5 s)")
    p.add_argument("--pair", action="store_true",
                   help="also run the aggressive cond/uncond pair: B=2, N=75600, 40x128 heads, "
                        "40 layers, T=40 {40,10,5} over 10/30/60%%, m=2 (~2-3 minutes, 124 GB "
                        "of caches)")
    p.add_argument("--sweep", action="store_true",
                   help="also time the large-head sweep: N=75600, 40x128 heads, active fraction "
                        "1, 1/2, 1/4, 1/8 (attention, selection, scatter, Euler per kernel)")
    p.add_argument("--split", action="store_true",
                   help="also time attention with and without the split-key workspace on the "
                        "shapes whose last round of query tiles leaves compute units idle, and "
                        "the pair's dense launch over the same cache (included in --sweep)")
    p.add_argument("--proj", action="store_true",
                   help="also time the fused QKV projection with the cache write "
                        "(hsa_qkv_project) against library linear + hsa_kv_update")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 512 MiB device copy 3 times (reference for HBM counters)")
    return p.parse_args()


def copy_calibration(torch):
    """A plain copy of known size: 512 MiB read + 512 MiB written per launch.  Under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives the counters' scale on this GPU."""
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4,
                      "launches": 3}))


def attn_source_hash() -> str:
    import importlib.util
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        # code only: a comment edit does not invalidate the counters
        code = [ln.split("//", 1)[0].rstrip() for ln in open(f, encoding="utf-8").read().splitlines()]
        h.update("\n".join(ln for ln in code if ln).encode())
    spec = importlib.util.spec_from_file_location(
        "attn_loop_gen", os.path.join(ROOT, "sparse_attention_l1_amd", "csrc", "attn_loop_gen.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    h.update("\n".join(gen.generate(True) + gen.generate(False)).encode())
    h.update(gen.clobber_list().encode())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary, or None when
    the summary is missing or was taken on a different version of the kernel source."""
    if not os.path.exists(ATTN_PMC_SUMMARY):
        return None
    text = open(ATTN_PMC_SUMMARY).read()
    h = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != attn_source_hash():
        return None
    return float(t.group(1))


class SingleStep:
    """Device state of the single-step workload and one call per path step."""

    def __init__(self, hs, synth, torch):
        self.hs, self.torch = hs, torch
        cfg = synth.single_step()
        self.cfg = cfg
        N, C, H, D = cfg.n_tokens, cfg.channels, cfg.heads, cfg.head_dim
        dev = torch.device("cuda")
        vm = synth.VelocityModel(cfg)
        src = synth.QKVSource(cfg)
        na = hs.hsastep_n_active(N, cfg.budgets, cfg.sizes, cfg.T, cfg.m, cfg.iteration)
        self.na = na
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        bits = lambda a: up(np.ascontiguousarray(a).view(np.int16))
        self.v_prev, self.v_cur = up(vm.v_prev), up(vm(0))
        self.v_model = up(vm(cfg.iteration))           # the model's velocity at this iteration
        self.x = up(synth.latent0(cfg))
        self.v_hat = self.v_prev.clone()
        pre = src.prefill(0)
        self.k_cache, self.v_cache = bits(pre), bits(pre)
        self.q = bits(src.rows("q", 0, cfg.iteration, na))
        self.k_new = bits(src.rows("k", 0, cfg.iteration, na))
        self.v_new = bits(src.rows("v", 0, cfg.iteration, na))
        self.out = torch.empty_like(self.q)
        self.group_id = torch.empty(N, dtype=torch.int32, device=dev)
        self.active_idx = torch.empty(N, dtype=torch.int32, device=dev)
        self.active_pos = torch.empty(N, dtype=torch.int32, device=dev)
        self.x_act = torch.empty((N, C), dtype=torch.float32, device=dev)
        self.v_fresh = torch.empty((na, C), dtype=torch.float32, device=dev)
        self.ws = hs.workspace(N, cfg.n_groups, dev)
        self.attn_ws = hs.attention_workspace(na, N, cfg.batch, H, D, dev)
        sig = np.linspace(1.0, 0.0, cfg.T + 1, dtype=np.float64).astype(np.float32)
        self.s_cur, self.s_next = float(sig[cfg.iteration]), float(sig[cfg.iteration + 1])
        self.scale = float(np.float32(1.0 / np.sqrt(D)))
        self.flops = 4.0 * cfg.batch * na * N * H * D

    def step(self, ev=None):
        hs, c = self.hs, self.cfg
        hs.hsa_select_groups(self.v_prev, self.v_cur, c.sizes, self.group_id, None, self.ws)
        # the active set and the model's input rows (the active tokens' latent rows)
        na = hs.hsa_active_set_gather(self.group_id, c.budgets, c.sizes, c.T, c.m, c.iteration,
                                      self.active_idx, self.active_pos, self.x, self.x_act,
                                      self.ws)
        hs.hsastep_gather_rows(self.v_fresh, self.v_model, self.active_idx, na)  # model stand-in
        hs.hsa_kv_update(self.k_cache, self.v_cache, self.k_new, self.v_new, self.active_idx, na)
        if ev is not None:
            ev[0].record()
        hs.hsa_attention_active_ws(self.q, self.k_cache, self.v_cache, self.out, self.scale,
                                   self.attn_ws)
        if ev is not None:
            ev[1].record()
        hs.hsa_euler_step(self.x, self.v_hat, self.v_fresh, self.active_pos, na, self.s_cur,
                          self.s_next)


def _event_ms(torch, fn, reps, flush=None):
    """Mean GPU ms per call, from an event pair around each call.  Warm: the calls queue
    behind a ~2 ms spin of the GPU, so the host enqueues them all before the GPU reaches them
    and the gap between consecutive calls is the GPU's own; the data stays in the caches.
    Cold: each call runs after a read of a 1 GiB buffer, which evicts the 256 MB infinity
    cache with clean lines, so its inputs come from HBM."""
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    if flush is None:
        torch.cuda._sleep(4_000_000)
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def run_mfma_ceiling(hs, synth, torch, attn_tflops, rounds=2000, reps=12):
    """The sustained rate of the attention kernel's MFMA (32x32x16 bf16) with nothing else in
    the loop, from the library's probe: 1024 workgroups of 4 wavefronts, 64 * rounds
    independent MFMAs per wavefront, about 20 ms per launch.  The first launches run while the
    chip's clock settles under the load, so the figure is the median of the last 8.  Finite
    operands (seeded, |x| in [0.25, 2)) give the ceiling an MFMA-bound kernel can reach; zero
    operands draw less power and give the optimistic one."""
    r = np.random.default_rng(7)
    vals = (r.uniform(0.25, 2.0, hs.MFMA_PROBE_OPERANDS)
            * r.choice([-1.0, 1.0], hs.MFMA_PROBE_OPERANDS)).astype(np.float32)
    finite = torch.from_numpy(synth.f32_to_bf16_bits(vals).view(np.int16)).cuda()
    zeros = torch.zeros_like(finite)
    workgroups = 1024
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    out = {"instruction": "v_mfma_f32_32x32x16_bf16", "workgroups": workgroups,
           "mfmas_per_wave": 64 * rounds}
    for tag, ops in (("finite_operands", finite), ("zero_operands", zeros)):
        flops = 0.0
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record()
            flops = hs.hsastep_mfma_probe(ops, sink, rounds, workgroups)
            b.record()
        torch.cuda.synchronize()
        rates = [flops / (a.elapsed_time(b) * 1e-3) / 1e12 for a, b in evs]
        out[tag + "_tflops"] = float(np.median(rates[-8:]))
        if tag == "finite_operands" and not np.isfinite(sink.cpu().numpy()).all():
            raise RuntimeError("mfma probe produced a non-finite sum")
    out["attention_frac_of_finite_ceiling"] = attn_tflops / out["finite_operands_tflops"]
    return out


def run_streaming(hs, synth, torch, st, reps=20):
    """The HBM-bound steps one by one: per call, microseconds, algorithmic bytes and the
    fraction of 8 TB/s, at the single-step sizes (warm: back-to-back calls, the figure the
    kernel trace of the single-step sequence gives) and from HBM (cold); Euler and the score
    also at the large-head sweep size (N = 75600, from HBM); and the floor of a launch that
    moves 16 bytes.  The selection and the active set are latency bound (several dependent
    launches over 4N-byte arrays) and are reported in microseconds."""
    dev = torch.device("cuda")
    c = st.cfg
    N, C, H, D, na = c.n_tokens, c.channels, c.heads, c.head_dim, st.na
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)
    flush = lambda: torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)
    one_idx = torch.zeros(1, dtype=torch.int32, device=dev)
    tiny_src = torch.zeros((1, 4), dtype=torch.float32, device=dev)
    tiny_dst = torch.empty_like(tiny_src)
    out = {"peak_gbs": PEAK_HBM_GBS, "kernels": {}}

    def entry(name, fn, nbytes, cold=True):
        e = {"us_warm": _event_ms(torch, fn, reps) * 1e3}
        if cold:
            e["us_cold"] = _event_ms(torch, fn, max(reps // 2, 5), flush) * 1e3
        if nbytes:
            e["bytes"] = nbytes
            for k in ("warm", "cold"):
                if f"us_{k}" in e:
                    e[f"gbs_{k}"] = nbytes / e[f"us_{k}"] / 1e3
                    e[f"frac_{k}"] = e[f"gbs_{k}"] / PEAK_HBM_GBS
        out["kernels"][name] = e

    entry("launch_floor (gather of one 16-byte row)",
          lambda: hs.hsastep_gather_rows(tiny_dst, tiny_src, one_idx, 1), 0)
    entry("kv_update", lambda: hs.hsa_kv_update(st.k_cache, st.v_cache, st.k_new, st.v_new,
                                                st.active_idx, na),
          4.0 * c.batch * na * H * D * 2 + 4 * na)
    entry("gather_rows (active latent rows)",
          lambda: hs.hsastep_gather_rows(st.x_act, st.x, st.active_idx, na), 2.0 * na * C * 4 + 4 * na)
    entry("euler_step", lambda: hs.hsa_euler_step(st.x, st.v_hat, st.v_fresh, st.active_pos, na,
                                                  st.s_cur, st.s_next),
          3.0 * N * C * 4 + na * C * 4 + 4 * N)
    entry("select_groups (score + 4 grouping launches)",
          lambda: hs.hsa_select_groups(st.v_prev, st.v_cur, c.sizes, st.group_id, None, st.ws),
          2.0 * N * C * 4 + 4 * N)
    entry("active_set_gather (2 launches, with the active latent rows)",
          lambda: hs.hsa_active_set_gather(st.group_id, c.budgets, c.sizes, c.T, c.m, c.iteration,
                                           st.active_idx, st.active_pos, st.x, st.x_act, st.ws),
          2.0 * na * C * 4 + 8.0 * N + 4 * na)
    entry("active_set (2 launches)",
          lambda: hs.hsa_active_set(st.group_id, c.budgets, c.sizes, c.T, c.m, c.iteration,
                                    st.active_idx, st.active_pos, st.ws), 0)
    # the large-head sweep's latent (N = 75600, 64 channels, half the tokens active), from HBM
    N4 = 75600
    g = torch.Generator(device=dev).manual_seed(20260512)
    x4 = torch.randn((N4, C), device=dev, generator=g)
    vh4 = torch.randn((N4, C), device=dev, generator=g)
    vc4 = torch.randn((N4, C), device=dev, generator=g)
    na4 = N4 // 2
    pos4 = torch.full((N4,), -1, dtype=torch.int32, device=dev)
    pos4[::2] = torch.arange(na4, dtype=torch.int32, device=dev)
    vf4 = torch.randn((na4, C), device=dev, generator=g)
    g4 = torch.empty(N4, dtype=torch.int32, device=dev)
    ws4 = hs.workspace(N4, 1, dev)
    entry("euler_step N=75600", lambda: hs.hsa_euler_step(x4, vh4, vf4, pos4, na4, 0.875, 0.85),
          3.0 * N4 * C * 4 + na4 * C * 4 + 4 * N4)
    entry("select_groups K=1 N=75600 (score + assignment)",
          lambda: hs.hsa_select_groups(vh4, vc4, (N4,), g4, None, ws4), 2.0 * N4 * C * 4 + 4 * N4)
    # plain device copy (torch copy_) moving the same byte counts, and 1 GiB: the ceiling a
    # streaming kernel of that size can reach
    copies = {}
    for moved in (16.9e6, 29.5e6, 68.0e6, 201.3e6, 2 ** 31):
        n = int(moved / 8)
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        us_w = _event_ms(torch, lambda: b.copy_(a), reps) * 1e3
        us_c = _event_ms(torch, lambda: b.copy_(a), 5, flush) * 1e3
        copies[f"{moved / 1e6:.1f} MB"] = {"us_warm": us_w, "us_cold": us_c,
                                           "gbs_warm": 8.0 * n / us_w / 1e3,
                                           "gbs_cold": 8.0 * n / us_c / 1e3}
        del a, b
    out["copy_ceiling"] = copies
    # the library's own row copy (hsastep_gather_rows with the identity index, 256-byte rows)
    own = {}
    for moved in (29.5e6, 68.0e6, 201.3e6, 2 ** 31):
        rows = int(moved / 2 / 256)
        a = torch.ones((rows, 64), dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        idx = torch.arange(rows, dtype=torch.int32, device=dev)
        fn = lambda: hs.hsastep_gather_rows(b, a, idx, rows)
        us_c = _event_ms(torch, fn, 5, flush) * 1e3
        own[f"{moved / 1e6:.1f} MB"] = {"us_cold": us_c, "gbs_cold": 2.0 * rows * 256 / us_c / 1e3}
        del a, b, idx
    out["row_copy_ceiling"] = own
    del flush_buf
    return out


def cpu_baseline(budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload: the full selection,
    active set, KV scatter and Euler update, plus attention for a sample of active query rows
    (all heads), extrapolated linearly to all |A| rows (every row costs the same)."""
    import oracle
    from sparse_attention_l1_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cfg = synth.single_step()
    vm = synth.VelocityModel(cfg)
    src = synth.QKVSource(cfg)
    i = cfg.iteration
    vp, vc = vm.v_prev, vm(0)
    x0 = synth.latent0(cfg)
    v_model = vm(i)
    t0 = time.perf_counter()
    g, _ = oracle.select_groups(vp, vc, cfg.sizes)
    idx, pos = oracle.active_set(g, cfg.budgets, cfg.T, cfg.m, i)
    na = idx.shape[0]
    x0[idx]                      # gather of the active rows (model input)
    pre = src.prefill(0)
    kc, vcache = pre.copy(), pre.copy()
    kn, vn, q = (src.rows(t, 0, i, na) for t in ("k", "v", "q"))
    oracle.kv_update(kc, vcache, kn, vn, idx)
    oracle.euler_step(x0, vp, v_model[idx], idx, np.float32(0.875), np.float32(0.85))
    t_rest = time.perf_counter() - t0
    scale = float(np.float32(1.0 / np.sqrt(cfg.head_dim)))
    # attention on seeded samples of active query rows, grown until the CPU budget is used
    order = synth.sample_rows(cfg.cfg_id, na, na, tag=1)
    rows, t_attn_s, chunk = 0, 0.0, 64
    while rows < na and t_rest + t_attn_s < budget_s:
        sel = np.sort(order[rows:rows + chunk])
        t2 = time.perf_counter()
        oracle.attention_active(q[:, sel], kc, vcache, scale)
        t_attn_s += time.perf_counter() - t2
        rows += sel.size
        chunk = min(chunk * 2, 2048)
    t_attn = t_attn_s * na / rows
    t_step = t_rest + t_attn
    flops = 4.0 * na * cfg.n_tokens * cfg.heads * cfg.head_dim
    return {"value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"single step N=32760: selection, active set, KV scatter and Euler in full; "
                       f"attention for {rows} of {na} active query rows x 12 heads, "
                       f"extrapolated linearly; {t_rest + t_attn_s:.1f} s of CPU time, "
                       f"extrapolated step {t_step:.1f} s")}


def _timed_calls(hs, torch, names):
    """Wraps the named entry points of the binding module so that every call is bracketed by a
    HIP event pair on the current stream; returns (restore, records) with records[name] a list
    of event pairs.  Used for one extra pass of a loop only: the events add a little work."""
    records = {n: [] for n in names}
    orig = {n: getattr(hs, n) for n in names}

    def wrap(n):
        f = orig[n]

        def call(*a, **k):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            r = f(*a, **k)
            e1.record()
            records[n].append((e0, e1))
            return r
        return call

    for n in names:
        setattr(hs, n, wrap(n))

    def restore():
        for n in names:
            setattr(hs, n, orig[n])
    return restore, records


def run_loop(hs, synth, torch, cfg, reps=1, breakdown=False):
    """Whole sampling runs (all T iterations, every layer) through the C ABI with the synthetic
    model stand-in (seeded Q/K/V pool windows and velocities, on the device): ms per iteration
    (HIP events around each) over `reps` runs from the same initial state, and the attention
    FLOPs of a run over its wall time.  With breakdown, one more run times every entry point
    call (events around each) and reports ms per iteration per entry point."""
    from sparse_attention_l1_amd.sampler import HsaSampler
    dev = torch.device("cuda")
    N, C, H, D, B = cfg.n_tokens, cfg.channels, cfg.heads, cfg.head_dim, cfg.batch
    src = synth.QKVSource(cfg)
    vm = synth.VelocityModel(cfg)
    pools = {t: torch.from_numpy(src.pools[t].bits.view(np.int16)).to(dev) for t in "qkv"}
    pre = torch.from_numpy(src.prefill(0).view(np.int16)).to(dev)
    del src.prefill_pool
    v_all = [torch.from_numpy(vm(i)).to(dev) for i in range(cfg.T)]
    x0 = torch.from_numpy(synth.latent0(cfg)).to(dev)
    vp = torch.from_numpy(vm.v_prev).to(dev)

    class PoolModel:
        def qkv(self, l, i, active_idx, na):
            need = na * H * D
            wins = lambda t: [pools[t][src.pools[t].offset(need, b, l, i):][:need] for b in range(B)]
            if B == 1:
                return tuple(wins(t)[0].view(1, na, H, D) for t in "qkv")
            return tuple(torch.stack(wins(t)).view(B, na, H, D) for t in "qkv")

        def velocity(self, i, active_idx, na):
            out = vbuf[:na]
            hs.hsastep_gather_rows(out, v_all[i], active_idx, na)
            return out

    vbuf = torch.empty((N, C), dtype=torch.float32, device=dev)
    smp = HsaSampler(n_tokens=N, channels=C, batch=B, heads=H, head_dim=D, layers=cfg.layers,
                     T=cfg.T, budgets=cfg.budgets, group_sizes=cfg.sizes, m=cfg.m)
    model = PoolModel()

    def one_run(tag):
        smp.reset(x0, vp, lambda l: (pre, pre))
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(cfg.T)]
        flops = 0.0
        t0 = time.perf_counter()
        for i in range(cfg.T):
            evs[i][0].record()
            smp.iteration(i, model)
            evs[i][1].record()
            flops += 4.0 * B * smp.n_active * N * H * D * cfg.layers
            if B > 1 or cfg.layers > 30:
                torch.cuda.synchronize()   # long iterations: report progress as they finish
                print(f"bench: {cfg.name}{tag}: iteration {i} done, |A| = {smp.n_active}",
                      file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return [a.elapsed_time(b) for a, b in evs], flops, wall

    runs = []
    for r in range(reps):
        runs.append(one_run(f" run {r + 1}/{reps}"))
        print(f"bench: {cfg.name}: run {r + 1}/{reps}: {np.mean(runs[-1][0]):.2f} ms per iteration",
              file=sys.stderr, flush=True)
    per_iter = np.mean([r[0] for r in runs], axis=0)
    flops = runs[0][1]
    wall = float(np.mean([r[2] for r in runs]))
    out = {"workload": cfg.name, "iterations": cfg.T, "layers": cfg.layers, "batch": B,
           "runs": reps,
           "ms_per_iteration_mean": float(np.mean(per_iter)),
           "ms_per_iteration_mean_per_run": [round(float(np.mean(r[0])), 3) for r in runs],
           "ms_per_iteration": [round(float(x), 3) for x in per_iter],
           "ms_total": float(np.sum(per_iter)),
           "attention_pflop": flops / 1e15, "tflops_effective": flops / wall / 1e12,
           "wall_s": wall}
    if breakdown:
        names = ["hsa_select_groups", "hsa_active_set_gather", "hsastep_gather_rows",
                 "hsa_kv_update", "hsa_attention_active_ws", "hsa_euler_step"]
        restore, rec = _timed_calls(hs, torch, names)
        try:
            t_iter, _, _ = one_run(" (per entry point)")
        finally:
            restore()
        per = {n: sum(a.elapsed_time(b) for a, b in rec[n]) / cfg.T for n in names}
        out["per_entry_point_ms_per_iteration"] = {
            "note": "one extra run with HIP events around every call (the model's velocity rows "
                    "come from hsastep_gather_rows, a stand-in for the model)",
            "ms_per_iteration_of_that_run": float(np.mean(t_iter)),
            **{n: round(v, 4) for n, v in per.items()}}
    return out


def run_proj(hs, torch, reps=10):
    """Fused QKV projection of the active rows with the cache write in its epilogue
    (hsa_qkv_project), against the unfused pair: torch's linear (hipBLASLt) into a [|A|, 3HD]
    buffer, then hsa_kv_update of its K/V parts.  Seeded N(0,1) bf16 inputs on the device;
    model dim = H * D; HIP events around each call (mean of reps after one warm-up)."""
    dev = torch.device("cuda")
    out = {"workload": "QKV projection of the active rows + cache write", "points": []}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for name, B, A, N, H, D in (("single step", 1, 16380, 32760, 12, 128),
                                ("large-head sweep f=0.5", 1, 37800, 75600, 40, 128),
                                ("aggressive pair, 10% active", 2, 7560, 75600, 40, 128)):
        HD, Dm = H * D, H * D
        gen = torch.Generator(device=dev).manual_seed(20260512)
        x = torch.randn((B, A, Dm), device=dev, generator=gen).to(torch.bfloat16)
        w = (torch.randn((3 * HD, Dm), device=dev, generator=gen) / Dm ** 0.5).to(torch.bfloat16)
        bias = torch.zeros(3 * HD, device=dev, dtype=torch.bfloat16)
        kc = torch.zeros((B, N, H, D), device=dev, dtype=torch.bfloat16)
        vc = torch.zeros_like(kc)
        idx = torch.from_numpy(np.sort(np.random.default_rng(0).choice(N, A, replace=False))
                               .astype(np.int32)).to(dev)
        q = torch.empty((B, A, H, D), device=dev, dtype=torch.bfloat16)
        flops = 2.0 * B * A * Dm * 3 * HD

        def unfused():
            y = torch.nn.functional.linear(x, w, bias)
            kn = y[..., HD:2 * HD].contiguous().view(B, A, H, D)
            vn = y[..., 2 * HD:].contiguous().view(B, A, H, D)
            hs.hsa_kv_update(kc, vc, kn, vn, idx, A)

        t_f = timed(lambda: hs.hsa_qkv_project(x, w, bias, q, kc, vc, idx, A))
        t_u = timed(unfused)
        t_l = timed(lambda: torch.nn.functional.linear(x, w, bias))
        out["points"].append({"shape": name, "batch": B, "n_active": A, "n_tokens": N,
                              "model_dim": Dm, "out_dim": 3 * HD, "gflop": flops / 1e9,
                              "fused_ms": t_f, "fused_tflops": flops / t_f / 1e9,
                              "fused_frac_of_bf16_peak": flops / t_f / 1e9 / PEAK_BF16_TFLOPS,
                              "unfused_ms": t_u, "library_linear_ms": t_l,
                              "library_linear_tflops": flops / t_l / 1e9})
        print(f"bench: projection {name}: fused {t_f:.3f} ms, unfused {t_u:.3f} ms", file=sys.stderr,
              flush=True)
    return out


def run_split_gain(hs, torch, reps=5):
    """Attention with and without the workspace in the same run, for the shapes whose last
    round of query tiles leaves compute units idle: the full schedule at 25% and 75% active,
    the aggressive pair at 10%, the sweep at f = 1 and 1/4 (seeded N(0,1) data, one layer).
    For the pair, the dense launch (every token active) over the same cache is timed too, so
    that the 10%-active rate can be set against the dense rate of the same K/V stream."""
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"compute_units": cus, "points": []}
    gen = torch.Generator(device=dev).manual_seed(20260512)
    for name, B, A, N, H in (("full schedule, 25% active", 1, 8190, 32760, 12),
                             ("full schedule, 75% active", 1, 24570, 32760, 12),
                             ("aggressive pair, 10% active", 2, 7560, 75600, 40),
                             ("large-head sweep f=1", 1, 75600, 75600, 40),
                             ("large-head sweep f=1/4", 1, 18900, 75600, 40)):
        q = torch.randn((B, A, H, 128), device=dev, generator=gen).to(torch.bfloat16)
        kc = torch.randn((B, N, H, 128), device=dev, generator=gen).to(torch.bfloat16)
        vc = torch.randn((B, N, H, 128), device=dev, generator=gen).to(torch.bfloat16)
        o = torch.empty_like(q)
        ws = hs.attention_workspace(A, N, B, H, 128, dev)
        scale = float(np.float32(1.0 / np.sqrt(128)))
        flops = 4.0 * B * A * N * H * 128
        t_plain = _event_ms(torch, lambda: hs.hsa_attention_active(q, kc, vc, o, scale), reps)
        t_ws = _event_ms(torch, lambda: hs.hsa_attention_active_ws(q, kc, vc, o, scale, ws), reps)
        pt = {"shape": name, "batch": B, "n_active": A, "n_tokens": N, "heads": H,
              "plan": list(hs.hsastep_attention_plan(A, N, B, H, 128, cus, ws.numel())),
              "ms_without_workspace": t_plain, "ms_with_workspace": t_ws,
              "tflops_without": flops / t_plain / 1e9, "tflops_with": flops / t_ws / 1e9}
        print(f"bench: split {name}: {t_plain:.3f} -> {t_ws:.3f} ms", file=sys.stderr, flush=True)
        del q, o, ws
        if name.startswith("aggressive pair"):
            qd = torch.randn((B, N, H, 128), device=dev, generator=gen).to(torch.bfloat16)
            od = torch.empty_like(qd)
            wsd = hs.attention_workspace(N, N, B, H, 128, dev)
            t_dense = _event_ms(torch, lambda: hs.hsa_attention_active_ws(qd, kc, vc, od, scale, wsd), 2)
            fd = 4.0 * B * N * N * H * 128
            pt["dense_ms_same_cache"] = t_dense
            pt["dense_tflops_same_cache"] = fd / t_dense / 1e9
            pt["with_workspace_frac_of_dense"] = pt["tflops_with"] / pt["dense_tflops_same_cache"]
            pt["without_workspace_frac_of_dense"] = pt["tflops_without"] / pt["dense_tflops_same_cache"]
            print(f"bench: split {name}: dense over the same cache {t_dense:.3f} ms", file=sys.stderr,
                  flush=True)
            del qd, od, wsd
        out["points"].append(pt)
        del kc, vc
    return out


def run_sweep(hs, synth, torch, reps=5):
    """Large-head sweep (N=75600 on a 21x45x80 grid, 40 heads x 128, 64 channels): per active
    fraction f, each kernel of one iteration timed alone with HIP events (mean of reps; the
    KV update and the Euler update with the infinity cache flushed before each rep).
    Q/K/V and the cache are seeded N(0,1) values drawn on the device."""
    dev = torch.device("cuda")
    out = {"workload": "large-head sweep N=75600 21x45x80, 40x128, 1 layer", "points": []}
    gen = torch.Generator(device=dev).manual_seed(20260512)
    N, H, D = 75600, 40, 128
    kc = torch.randn((1, N, H, D), device=dev, generator=gen).to(torch.bfloat16)
    vc = torch.randn((1, N, H, D), device=dev, generator=gen).to(torch.bfloat16)
    scale = float(np.float32(1.0 / np.sqrt(D)))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # HBM-bound kernels: 1 GiB read before each rep evicts the 256 MB infinity cache with
    # clean lines, so their inputs come from HBM and no write-back of the flush competes;
    # only the kernel itself is inside the events
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)

    def timed_cold(fn):
        fn()
        total = 0.0
        for _ in range(reps):
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            total += a.elapsed_time(b)
        return total / reps

    for f in (1.0, 0.5, 0.25, 0.125):
        cfg = synth.sweep(f)
        C = cfg.channels
        vm = synth.VelocityModel(cfg)
        vp = torch.from_numpy(vm.v_prev).to(dev)
        vcur = torch.from_numpy(vm(0)).to(dev)
        g = torch.empty(N, dtype=torch.int32, device=dev)
        idx = torch.empty(N, dtype=torch.int32, device=dev)
        pos = torch.empty(N, dtype=torch.int32, device=dev)
        ws = hs.workspace(N, cfg.n_groups, dev)
        hs.hsa_select_groups(vp, vcur, cfg.sizes, g, None, ws)
        na = hs.hsa_active_set(g, cfg.budgets, cfg.sizes, cfg.T, cfg.m, cfg.iteration, idx, pos, ws)
        q = torch.randn((1, na, H, D), device=dev, generator=gen).to(torch.bfloat16)
        kn = torch.randn((1, na, H, D), device=dev, generator=gen).to(torch.bfloat16)
        vn = torch.randn((1, na, H, D), device=dev, generator=gen).to(torch.bfloat16)
        o = torch.empty_like(q)
        x = torch.from_numpy(synth.latent0(cfg)).to(dev)
        vh = vp.clone()
        vf = torch.empty((na, C), dtype=torch.float32, device=dev)
        hs.hsastep_gather_rows(vf, vcur, idx, na)
        flops = 4.0 * na * N * H * D
        aws = hs.attention_workspace(na, N, 1, H, D, dev)
        t_att = timed(lambda: hs.hsa_attention_active_ws(q, kc, vc, o, scale, aws))
        t_sel = timed(lambda: hs.hsa_select_groups(vp, vcur, cfg.sizes, g, None, ws))
        t_act = timed(lambda: hs.hsa_active_set(g, cfg.budgets, cfg.sizes, cfg.T, cfg.m,
                                                cfg.iteration, idx, pos, ws))
        t_kv = timed_cold(lambda: hs.hsa_kv_update(kc, vc, kn, vn, idx, na))
        t_eu = timed_cold(lambda: hs.hsa_euler_step(x, vh, vf, pos, na, 0.875, 0.85))
        kv_bytes = 4.0 * na * H * D * 2 + 4 * na
        eu_bytes = 3.0 * N * C * 4 + na * C * 4 + 4 * N
        out["points"].append({
            "active_fraction": f, "n_active": na,
            "attention_ms": t_att, "attention_tflops": flops / t_att / 1e9,
            "attention_frac_of_bf16_peak": flops / t_att / 1e9 / PEAK_BF16_TFLOPS,
            "select_groups_us": t_sel * 1e3, "active_set_us": t_act * 1e3,
            "kv_update_us": t_kv * 1e3, "kv_update_gbs": kv_bytes / t_kv / 1e6,
            "euler_us": t_eu * 1e3, "euler_gbs": eu_bytes / t_eu / 1e6})
        print(f"bench: sweep f={f} attention {flops / t_att / 1e9:.0f} TFLOP/s", file=sys.stderr,
              flush=True)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the HSA path is built and "
              f"timed on a single MI355X; sharding across GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_l1_amd import hsastep as hs
    from sparse_attention_l1_amd import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    print("bench: building single-step inputs", file=sys.stderr, flush=True)
    st = SingleStep(hs, synth, torch)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    print("bench: timing", file=sys.stderr, flush=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        st.step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    achieved = st.flops / (attn_ms * 1e-3) / 1e12
    traffic = load_traffic()
    res = {
        "metric": "HSA active-query attention TFLOP/s + ms per denoise iteration at N=32760",
        "value": st.flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V and cache, lognormal-drift fp32 velocities)",
        "config": {"workload": st.cfg.name, "n_tokens": st.cfg.n_tokens, "n_active": st.na,
                   "heads": st.cfg.heads, "head_dim": st.cfg.head_dim,
                   "channels": st.cfg.channels, "batch": st.cfg.batch,
                   "groups": {"budgets": list(st.cfg.budgets), "sizes": list(st.cfg.sizes),
                              "T": st.cfg.T, "m": st.cfg.m, "iteration": st.cfg.iteration}},
        "attention_ms_per_launch": attn_ms,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
    }
    if not args.no_mfma_ceiling:
        print("bench: sustained MFMA ceiling", file=sys.stderr, flush=True)
        res["mfma_ceiling"] = run_mfma_ceiling(hs, synth, torch, achieved)
    if not args.no_streaming:
        print("bench: streaming kernels and copy ceiling", file=sys.stderr, flush=True)
        res["streaming_kernels"] = run_streaming(hs, synth, torch, st)
    if not args.no_loop:
        print("bench: full schedule loop", file=sys.stderr, flush=True)
        res["full_schedule"] = run_loop(hs, synth, torch, synth.full_schedule(), reps=3,
                                        breakdown=True)
    if args.pair:
        print("bench: aggressive pair loop", file=sys.stderr, flush=True)
        res["aggressive_pair"] = run_loop(hs, synth, torch, synth.aggressive_pair())
    if args.proj:
        print("bench: fused QKV projection", file=sys.stderr, flush=True)
        res["qkv_projection"] = run_proj(hs, torch)
    if args.sweep:
        print("bench: large-head sweep", file=sys.stderr, flush=True)
        res["large_head_sweep"] = run_sweep(hs, synth, torch)
    if args.sweep or args.split:
        print("bench: split-key attention", file=sys.stderr, flush=True)
        res["attention_split_gain"] = run_split_gain(hs, torch)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
