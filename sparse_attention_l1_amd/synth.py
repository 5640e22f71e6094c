"""Seeded synthetic inputs for the HSA denoise-iteration path.

This module is the only code shared by the HIP path's callers (tests, bench) and
the CPU oracle's callers.  It draws random numbers and lays them out; it holds
none of the method's arithmetic (no scores, ranks, schedules, attention or
integration).  Everything is numpy on the host; callers upload what they need.

Workload shapes follow the HSA pages' setting (video DiTs such as Wan-2.1 /
Wan-2.2 / LTX-2 on 81-frame clips, "Technische Samenvatting: Heterogene
Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §4): the latent grids
21x30x52 and 21x45x80 correspond to 480x832 and 720x1280 video after the usual
4x temporal / 8x spatial VAE compression and 1x2x2 patching.  No model weights
or prompts are involved: velocities and Q/K/V rows are random stand-ins with
the statistics described below.

Seeds: ``rng(cfg_id, stream, *sub)`` = numpy default_rng on
SeedSequence([20260512, cfg_id, stream, *sub]).  Streams:
  0 initial latent x_0          1 previous velocity v_prev      2 drift scale lambda
  3 velocity noise z(i)         4/5/6 Q/K/V pools               7 cache prefill pool
  8 parity sample rows
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import concurrent.futures

import numpy as np

SEED = 20260512

STREAM_X0, STREAM_VPREV, STREAM_LAMBDA, STREAM_Z = 0, 1, 2, 3
STREAM_Q, STREAM_K, STREAM_V, STREAM_PREFILL, STREAM_SAMPLE = 4, 5, 6, 7, 8


def rng(cfg_id: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, cfg_id, stream, *sub]))


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    n_tokens N, channels C (latent channels per token), batch B (sequences that
    share one latent, e.g. a cond/uncond pair), heads H, head_dim D, layers L,
    T iterations, per-group step budgets s_k and token counts n_k, window m.
    ``iteration`` is the measured iteration of single-step workloads.
    """
    name: str
    cfg_id: int
    n_tokens: int
    channels: int
    batch: int
    heads: int
    head_dim: int
    layers: int
    T: int
    budgets: Tuple[int, ...]
    sizes: Tuple[int, ...]
    m: int
    drift: str = "lognormal"          # or "student_t3"
    iteration: Optional[int] = None
    grid: Optional[Tuple[int, int, int]] = None

    @property
    def n_groups(self) -> int:
        return len(self.budgets)


def tiny() -> Config:
    return Config("tiny N=256 4x8x8, 2x64, T=8 {8,4} m=1", 0, 256, 16, 1, 2, 64, 1,
                  8, (8, 4), (128, 128), 1, grid=(4, 8, 8))


def single_step() -> Config:
    """N=32760 (21x30x52), 12x128 heads, half the tokens active.

    Half of the tokens active by L1 relative change is realised as two groups
    {40, 20} of equal size at T=40, m=4, measured at iteration 5 (odd, outside
    both windows), where exactly the full-budget group is active.
    """
    return Config("single step N=32760 21x30x52, 12x128, 50% active", 1, 32760, 64, 1, 12,
                  128, 1, 40, (40, 20), (16380, 16380), 4, iteration=5, grid=(21, 30, 52))


def full_schedule() -> Config:
    return Config("full schedule N=32760, 12x128, 30 layers, T=40 {40,20,10,5} m=4", 2,
                  32760, 64, 1, 12, 128, 30, 40, (40, 20, 10, 5), (8190,) * 4, 4,
                  grid=(21, 30, 52))


def sweep(frac: float) -> Config:
    n = 75600
    if frac >= 1.0:
        budgets, sizes = (40,), (n,)
    else:
        a = int(round(frac * n))
        budgets, sizes = (40, 20), (a, n - a)
    return Config(f"large-head sweep N=75600 21x45x80, 40x128, f={frac}", 3, n, 64, 1, 40,
                  128, 40, 40, budgets, sizes, 4, iteration=5, grid=(21, 45, 80))


def aggressive_pair() -> Config:
    return Config("aggressive pair B=2 N=75600, 40x128, T=40 {40,10,5} m=2", 4, 75600, 64, 2,
                  40, 128, 40, 40, (40, 10, 5), (7560, 22680, 45360), 2, drift="student_t3",
                  grid=(21, 45, 80))


# --------------------------------------------------------------------------- helpers

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns uint16 bits.

    Inputs are finite; this is a storage-format conversion of generated data.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24   # chunks bound the temporaries; finite inputs cannot overflow uint32 here
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = (c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return out


def splitmix64(x: int) -> int:
    """SplitMix64 finaliser (Steele, Lea, Flood 2014), used to place pool windows."""
    m = (1 << 64) - 1
    x = (x + 0x9E3779B97F4A7C15) & m
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


# --------------------------------------------------------------------------- latent / velocity

def latent0(cfg: Config) -> np.ndarray:
    return rng(cfg.cfg_id, STREAM_X0).standard_normal((cfg.n_tokens, cfg.channels), dtype=np.float32)


def velocity_prev(cfg: Config) -> np.ndarray:
    return rng(cfg.cfg_id, STREAM_VPREV).standard_normal((cfg.n_tokens, cfg.channels),
                                                        dtype=np.float32)


def drift_scale(cfg: Config) -> np.ndarray:
    """Per-token drift scale lambda_n: lognormal(0,1), or |Student-t(3)| (heavy tail)."""
    g = rng(cfg.cfg_id, STREAM_LAMBDA)
    if cfg.drift == "student_t3":
        lam = np.abs(g.standard_t(3, size=cfg.n_tokens))
    else:
        lam = g.lognormal(0.0, 1.0, size=cfg.n_tokens)
    return lam.astype(np.float32)


class VelocityModel:
    """Stand-in for the DiT's velocity prediction: v(i)_n = v_prev_n + lambda_n * z(i)_n.

    v(-1) is v_prev itself, so the tiny workload's (v_prev, v_cur) pair is (v(-1), v(0)).
    """

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.v_prev = velocity_prev(cfg)
        self.lam = drift_scale(cfg)

    def __call__(self, i: int) -> np.ndarray:
        if i < 0:
            return self.v_prev.copy()
        z = rng(self.cfg.cfg_id, STREAM_Z, i).standard_normal(self.v_prev.shape, dtype=np.float32)
        return (self.v_prev + self.lam[:, None] * z).astype(np.float32)


# --------------------------------------------------------------------------- Q/K/V pools

class Pool:
    """A seeded pool of N(0,1) values rounded to bf16; tensors are windows into it.

    A window for (tensor, b, layer, i) starts at splitmix64(key) mod (len - need),
    rounded down to a multiple of 8 elements (16 bytes).
    """

    def __init__(self, cfg_id: int, stream: int, length: int):
        self.cfg_id, self.stream, self.length = cfg_id, stream, int(length)
        vals = rng(cfg_id, stream).standard_normal(self.length, dtype=np.float32)
        self.bits = f32_to_bf16_bits(vals)

    def offset(self, need: int, *key: int) -> int:
        if need > self.length:
            raise ValueError(f"pool of {self.length} elements is smaller than {need}")
        span = self.length - need
        if span == 0:
            return 0
        h = self.cfg_id * 1000003 + self.stream
        for k in key:
            h = splitmix64((h * 0x100000001B3) ^ (int(k) & ((1 << 64) - 1)))
        return (splitmix64(h) % (span + 1)) // 8 * 8

    def window(self, need: int, *key: int) -> np.ndarray:
        o = self.offset(need, *key)
        return self.bits[o:o + need]


def pool_length(need_max: int) -> int:
    n = 1 << 16
    while n < need_max + (need_max >> 2) + 64:
        n <<= 1
    return n


class QKVSource:
    """Seeded Q / new-K / new-V rows for the active tokens, plus the cache prefill.

    Shapes: q, k_new, v_new [B, n_active, H, D] bf16 bits; prefill [B, N, H, D].
    """

    def __init__(self, cfg: Config, max_rows: Optional[int] = None):
        self.cfg = cfg
        rows = cfg.n_tokens if max_rows is None else max_rows
        row = cfg.heads * cfg.head_dim
        need = rows * row
        jobs = [("q", STREAM_Q, need), ("k", STREAM_K, need), ("v", STREAM_V, need),
                ("prefill", STREAM_PREFILL, cfg.n_tokens * row)]
        # the four pools are independent seeded streams: generate them concurrently
        with concurrent.futures.ThreadPoolExecutor(len(jobs)) as ex:
            made = list(ex.map(lambda j: Pool(cfg.cfg_id, j[1], pool_length(j[2])), jobs))
        self.pools = {j[0]: p for j, p in zip(jobs[:3], made[:3])}
        self.prefill_pool = made[3]

    def rows(self, tensor: str, layer: int, i: int, n_rows: int) -> np.ndarray:
        c = self.cfg
        need = n_rows * c.heads * c.head_dim
        out = np.empty((c.batch, n_rows, c.heads, c.head_dim), np.uint16)
        for b in range(c.batch):
            out[b] = self.pools[tensor].window(need, b, layer, i).reshape(n_rows, c.heads,
                                                                         c.head_dim)
        return out

    def prefill(self, layer: int) -> np.ndarray:
        c = self.cfg
        need = c.n_tokens * c.heads * c.head_dim
        out = np.empty((c.batch, c.n_tokens, c.heads, c.head_dim), np.uint16)
        for b in range(c.batch):
            out[b] = self.prefill_pool.window(need, b, layer).reshape(c.n_tokens, c.heads,
                                                                      c.head_dim)
        return out


def sample_rows(cfg_id: int, n: int, k: int, tag: int = 0) -> np.ndarray:
    """k distinct sorted row indices in [0, n) (parity sampling)."""
    k = min(k, n)
    return np.sort(rng(cfg_id, STREAM_SAMPLE, tag).choice(n, size=k, replace=False))
