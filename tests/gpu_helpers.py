"""Shared helpers of the GPU tests: host<->device moves and the synthetic model.

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
