"""Shared helpers of the GPU tests: host<->device moves, the synthetic model, the attention
tolerance check and the seeded velocity kinds.

The synthetic model stands in for the DiT (its projections and velocity head):
seeded Q/K/V rows for the active tokens and seeded velocities, uploaded from the
same host arrays the oracle reads.
"""
import numpy as np
import torch

from sparse_attention_l1_amd import synth


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device int16 tensor with the same bits."""
    return dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class SyntheticModel:
    """Model stand-in for HsaSampler: seeded rows per (layer, iteration)."""

    def __init__(self, cfg: synth.Config, hs):
        self.cfg, self.hs = cfg, hs
        self.src = synth.QKVSource(cfg)
        self.vm = synth.VelocityModel(cfg)
        # the pools on the device: a (tensor, b, layer, i) window is then a device slice
        self.pools = {t: bits_dev(self.src.pools[t].bits) for t in ("q", "k", "v")}

    def qkv(self, l, i, active_idx, na):
        c = self.cfg
        need = na * c.heads * c.head_dim
        out = []
        for t in ("q", "k", "v"):
            wins = [self.pools[t][self.src.pools[t].offset(need, b, l, i):][:need]
                    for b in range(c.batch)]
            out.append(torch.stack(wins).view(c.batch, na, c.heads, c.head_dim))
        return tuple(out)

    def velocity(self, i, active_idx, na):
        full = dev(self.vm(i))
        out = torch.empty((max(na, 1), self.cfg.channels), dtype=torch.float32, device="cuda")
        self.hs.hsastep_gather_rows(out, full, active_idx, na)
        return out[:na]

    def prefill(self, l):
        p = bits_dev(self.src.prefill(l))
        return p, p


# attention bar of the parity tests: max-abs against the float64 oracle, for every input
# (unit-variance and peaky softmaxes alike).  Rounding the output to bf16 alone errs by at most
# half an ulp, 2^-8 * |O| for |O| in [2^k, 2^(k+1)) with the ulp taken at 2^k (0.0156 just below
# |O| = 8); the kernels' normaliser is the sum of the same rounded P that weights V, so a key
# that dominates the softmax carries no rounding error of its own.
ATOL = 2e-2


def attn_close(got_bits, want, label):
    got = bf16_to_f64(got_bits)
    err = np.abs(got - want)
    mx = float(np.max(np.abs(want))) if want.size else 0.0
    worst = float(err.max()) if err.size else 0.0
    print(f"[{label}] attention max-abs err {worst:.3e}, max|O| {mx:.3e}", flush=True)
    assert worst <= ATOL


def velocities(kind, n, c, seed):
    r = np.random.default_rng(seed)
    vp = r.standard_normal((n, c)).astype(np.float32)
    if kind == "ties":
        vp = np.ones((n, c), np.float32)
        return vp, (vp * np.float32(1.25)).astype(np.float32)
    if kind == "levels":
        # r is exactly one of 4 values: long runs of equal keys across many workgroups
        vp = np.ones((n, c), np.float32)
        lv = np.array([0.0, 0.5, 1.0, 2.0], np.float32)[r.integers(0, 4, n)]
        return vp, (vp + lv[:, None]).astype(np.float32)
    if kind == "heavy":
        lam = np.abs(r.standard_t(3, n)).astype(np.float32)
    else:
        lam = r.lognormal(0, 1, n).astype(np.float32)
    vc = (vp + lam[:, None] * r.standard_normal((n, c)).astype(np.float32)).astype(np.float32)
    if kind == "special":
        vp[::7] = 0
        vc[::14] = 0                # 0/0 rows
        vc[3::11, 0] = np.nan       # NaN rows
        vc[5::13] = vp[5::13]       # zero change
        vp[6::17, :] *= np.float32(2.0 ** -130)   # denormal magnitudes
    return vp, vc
