"""Host-side driver of the HSA sampling loop over the C ABI.

One call of ``HsaSampler.iteration(i, model)`` is one denoise iteration of
Heterogeneous Step Allocation ("Technische Samenvatting: Heterogene
Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.1-§2.4):

    active set A_i          hsa_active_set_gather (|A_i| known on the host, no sync; the
                                                   active latent rows into x_active)
    per layer:  model(A_i) -> q, k_new, v_new for the active tokens
                hsa_kv_update         fresh K/V rows overwrite their cache slots
                hsa_attention_active_ws  active queries x all N cached rows
    model(A_i) -> fresh velocities of the active tokens
    (at iteration max(m,1)-1, where every token is active; with reselect=True also
     at every later iteration in which every token is active)
                hsa_select_groups     groups by L1 relative velocity change
    hsa_euler_step          cached Euler update of all N latents

The model (the DiT's projections and velocity head) is outside the path: it is
passed in as an object with ``qkv(layer, i, active_idx, n_active)`` and
``velocity(i, active_idx, n_active)`` returning device tensors.  All device
work is enqueued on the current stream; nothing here synchronises.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from . import hsastep as hs


def sigma_schedule(T: int) -> np.ndarray:
    """sigma_0 = 1 ... sigma_T = 0, linear, computed in float64 and stored as float32."""
    return np.linspace(1.0, 0.0, T + 1, dtype=np.float64).astype(np.float32)


class HsaSampler:
    def __init__(self, *, n_tokens: int, channels: int, batch: int, heads: int, head_dim: int,
                 layers: int, T: int, budgets: Sequence[int], group_sizes: Sequence[int], m: int,
                 softmax_scale: Optional[float] = None, device="cuda", reselect: bool = False):
        self.N, self.C, self.B, self.H, self.D, self.L = n_tokens, channels, batch, heads, head_dim, layers
        self.T, self.budgets, self.sizes, self.m = T, list(budgets), list(group_sizes), m
        self.scale = float(np.float32(1.0 / np.sqrt(head_dim))) if softmax_scale is None else softmax_scale
        self.device = torch.device(device)
        self.sigma = sigma_schedule(T)
        dev = self.device
        self.x = torch.empty((n_tokens, channels), dtype=torch.float32, device=dev)
        self.v_hat = torch.empty_like(self.x)
        self.group_id = torch.zeros(n_tokens, dtype=torch.int32, device=dev)
        self.score = torch.empty(n_tokens, dtype=torch.float32, device=dev)
        self.active_idx = torch.empty(n_tokens, dtype=torch.int32, device=dev)
        # the active tokens' latent rows in active order: the model's input at this iteration
        self.x_active = torch.empty_like(self.x)
        self.active_pos = torch.empty(n_tokens, dtype=torch.int32, device=dev)
        self.ws = hs.workspace(n_tokens, len(budgets), dev)
        shape = (batch, n_tokens, heads, head_dim)
        self.k_cache: List[torch.Tensor] = [torch.empty(shape, dtype=torch.bfloat16, device=dev)
                                            for _ in range(layers)]
        self.v_cache: List[torch.Tensor] = [torch.empty(shape, dtype=torch.bfloat16, device=dev)
                                            for _ in range(layers)]
        self.attn_out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        # lets attention split the key range of a last round of query tiles that would leave
        # compute units idle (iterations with few active tokens)
        self.attn_ws = hs.attention_workspace(n_tokens, n_tokens, batch, heads, head_dim, dev)
        self.n_active = n_tokens
        self.selection_iter = max(m, 1) - 1
        self.reselect = reselect

    def reset(self, x0: torch.Tensor, v_prev: torch.Tensor,
              prefill: Callable[[int], Sequence[torch.Tensor]]) -> None:
        """x <- x0, velocity cache <- v_prev, every token in the baseline group, caches <- prefill."""
        self.x.copy_(x0)
        self.v_hat.copy_(v_prev)
        self.group_id.zero_()
        for l in range(self.L):
            k, v = prefill(l)
            self.k_cache[l].copy_(k)
            self.v_cache[l].copy_(v)

    def select(self, v_prev: torch.Tensor, v_cur: torch.Tensor) -> None:
        hs.hsa_select_groups(v_prev, v_cur, self.sizes, self.group_id, self.score, self.ws)

    def active_set(self, i: int) -> int:
        self.n_active = hs.hsa_active_set_gather(self.group_id, self.budgets, self.sizes, self.T,
                                                 self.m, i, self.active_idx, self.active_pos,
                                                 self.x, self.x_active, self.ws)
        return self.n_active

    def attention_layer(self, l: int, q: torch.Tensor, k_new: torch.Tensor,
                        v_new: torch.Tensor) -> torch.Tensor:
        na = self.n_active
        out = self.attn_out.view(-1)[: self.B * na * self.H * self.D].view(self.B, na, self.H, self.D)
        hs.hsa_kv_update(self.k_cache[l], self.v_cache[l], k_new, v_new, self.active_idx, na)
        hs.hsa_attention_active_ws(q, self.k_cache[l], self.v_cache[l], out, self.scale,
                                   self.attn_ws)
        return out

    def euler(self, i: int, v_fresh: torch.Tensor) -> None:
        hs.hsa_euler_step(self.x, self.v_hat, v_fresh, self.active_pos, self.n_active,
                          float(self.sigma[i]), float(self.sigma[i + 1]))

    def iteration(self, i: int, model, on_attention=None) -> None:
        na = self.active_set(i)
        for l in range(self.L):
            q, k_new, v_new = model.qkv(l, i, self.active_idx, na)
            out = self.attention_layer(l, q, k_new, v_new)
            if on_attention is not None:
                on_attention(l, out)
        v_fresh = model.velocity(i, self.active_idx, na)
        regroup = self.m >= 1 and i == self.selection_iter
        regroup |= self.reselect and na == self.N and i >= self.selection_iter
        if regroup:
            # every token is active here, so v_fresh is in token order
            self.select(self.v_hat, v_fresh)
        self.euler(i, v_fresh)
