"""CPU oracle for one HSA denoise iteration and the full HSA sampling loop.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
path never does, and this module imports nothing from it (no shared kernels,
headers, helpers or constants).

Plain numpy, written for a reader to check against the pages by eye: no
blocking, fusion or reordering beyond what each definition states.  Attention
is evaluated in float64 from the bfloat16 inputs; the latent/velocity state is
float32 with the rounding points spelled out, as the method keeps it.

Pages (the method's only description):
  [HSA-nl]  "Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor
            Efficiënte Videogeneratie", gist.science/nl/paper/2605.06892
  [HSA-de]  "Not All Tokens Need 40 Steps: Heterogeneous Step Allocation in
            Diffusion Transformers for Efficient Video Generation",
            gist.science/de/paper/2605.06892 (title, lay explainer, German summary)

Readings taken where the pages are silent (each marked READING below):
  R1 L1 relative change = ||v_cur - v_prev||_1 / ||v_prev||_1 per token.
  R2 fp32 sums use a balanced contiguous pairwise tree (C zero-padded to 2^k).
  R3 r: IEEE fp32 divide; 0/0 -> 0, x/0 -> +inf, NaN -> +inf.
  R4 largest r -> G_1 (full budget); ties broken by ascending token index.
  R5 iteration index i is zero-based, 0..T-1.
  R6 the window and the periodic rule combine by union.
  R7 sigma: T+1 values linear 1 -> 0 computed in fp64, stored in fp32;
     dt = fp32(sigma_{i+1} - sigma_i); x <- fl(x + fl(dt * v)), no fused multiply-add.
  R8 attention: softmax(q k^T * scale) v over all N cache rows, no mask.
  R9 selection happens once, inside iteration max(m,1)-1, comparing the fresh
     velocities with the velocity cache before the Euler write (for m = 0 the
     caller supplies (v_prev, v_cur) and selects before iteration 0).
  R10 cache slot = token index; scatter precedes attention in every layer.
  R11 variant (run_hsa(reselect=True)), the fuller reading of dynamic selection:
     besides the selection of R9, the groups are recomputed the same way at every
     later iteration in which every token is active (|A_i| = N), from the velocity
     cache and that iteration's fresh velocities, before the Euler write.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- formats


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 (uint16 bit patterns) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- schedule


def sigma_schedule(T: int) -> np.ndarray:
    """READING R7: sigma_0 = 1 ... sigma_T = 0, linear, rounded to fp32."""
    return np.linspace(1.0, 0.0, T + 1, dtype=np.float64).astype(np.float32)


def check_budgets(budgets, T: int) -> None:
    """[HSA-nl §2.1]: every budget s_k divides T and the baseline group has s_1 = T."""
    if len(budgets) < 1:
        raise ValueError("need at least one group")
    if budgets[0] != T:
        raise ValueError("baseline group G_1 must have the full budget s_1 = T")
    for s in budgets:
        if s <= 0 or T % s != 0:
            raise ValueError(f"budget {s} does not divide T={T}")


def group_active(i: int, s_k: int, T: int, m: int) -> bool:
    """Is a token of a group with budget s_k active at iteration i?

    [HSA-nl §2.1]: active iff i mod (T/s_k) = 0 (s_1 = T gives every iteration).
    [HSA-nl §2.4]: the first and last m iterations are full passes for all tokens.
    READINGS R5 (zero-based i) and R6 (union).
    """
    return (i < m) or (i >= T - m) or (i % (T // s_k) == 0)


def active_set(group_id: np.ndarray, budgets, T: int, m: int, i: int):
    """A_i as an ascending index list, plus the inverse map (-1 for skipped tokens).

    Returns (active_idx int32 [|A_i|], active_pos int32 [N]).
    """
    check_budgets(budgets, T)
    g = np.asarray(group_id)
    flags = np.array([group_active(i, budgets[k], T, m) for k in range(len(budgets))])
    active = flags[g]
    active_idx = np.flatnonzero(active).astype(np.int32)
    active_pos = np.full(g.shape[0], -1, np.int32)
    active_pos[active_idx] = np.arange(active_idx.shape[0], dtype=np.int32)
    return active_idx, active_pos


def n_active(group_sizes, budgets, T: int, m: int, i: int) -> int:
    """|A_i| from the group sizes alone (every token of a group shares its schedule)."""
    return int(sum(n for n, s in zip(group_sizes, budgets) if group_active(i, s, T, m)))


# ----------------------------------------------------------------------------- selection


def tree_sum_rows(a: np.ndarray) -> np.ndarray:
    """READING R2: per-row fp32 sum by a balanced contiguous pairwise tree.

    Width is zero-padded to the next power of two; level by level, element j of
    the next level is (element 2j) + (element 2j+1), each addition rounded to fp32.
    """
    a = np.asarray(a, dtype=np.float32)
    w = a.shape[1]
    p = 1
    while p < w:
        p *= 2
    if p != w:
        a = np.concatenate([a, np.zeros((a.shape[0], p - w), np.float32)], axis=1)
    while a.shape[1] > 1:
        a = (a[:, 0::2] + a[:, 1::2]).astype(np.float32)
    return a[:, 0]


def l1_relative_change(v_prev: np.ndarray, v_cur: np.ndarray) -> np.ndarray:
    """Per-token L1 relative change of the velocity prediction ([HSA-nl §2.1],
    Dynamic Token Selection), READINGS R1-R3.  Returns r [N] float32, r >= +0."""
    v_prev = np.asarray(v_prev, dtype=np.float32)
    v_cur = np.asarray(v_cur, dtype=np.float32)
    num = tree_sum_rows(np.abs(v_cur - v_prev))
    den = tree_sum_rows(np.abs(v_prev))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (num / den).astype(np.float32)
    r = np.where(den == 0, np.where(num == 0, np.float32(0), np.float32(np.inf)), r)
    r = np.where(np.isnan(r), np.float32(np.inf), r).astype(np.float32)
    return r


def assign_groups(r: np.ndarray, group_sizes) -> np.ndarray:
    """Tokens ranked by r, fastest-changing first, fill G_1, G_2, ... in order.

    [HSA-nl §2 intro, §2.1]: slower-evolving tokens get fewer steps; G_1 keeps
    the full schedule.  READING R4: ties by ascending token index.
    The rank is a stable sort on the fp32 value itself (r >= +0, so its bit
    pattern orders the same way).
    """
    r = np.asarray(r, dtype=np.float32)
    n = r.shape[0]
    sizes = np.asarray(group_sizes, dtype=np.int64)
    if sizes.sum() != n or (sizes < 0).any():
        raise ValueError("group sizes must be non-negative and sum to N")
    key = r.view(np.uint32)
    order = np.lexsort((np.arange(n), ~key))          # key descending, index ascending
    rank = np.empty(n, np.int64)
    rank[order] = np.arange(n)
    bounds = np.cumsum(sizes)
    return np.searchsorted(bounds, rank, side="right").astype(np.int32)


def select_groups(v_prev, v_cur, group_sizes):
    """Dynamic Token Selection: returns (group_id int32 [N], r float32 [N])."""
    r = l1_relative_change(v_prev, v_cur)
    return assign_groups(r, group_sizes), r


# ----------------------------------------------------------------------------- KV cache + attention


def kv_update(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              active_idx: np.ndarray) -> None:
    """[HSA-nl §2.2, items 2-3]: fresh K/V rows of the active tokens overwrite
    their slots in the per-layer cache; skipped tokens keep their (stale but
    valid) rows.  Caches [B, N, H, D], new rows [B, |A|, H, D], in place."""
    k_cache[:, active_idx] = k_new
    v_cache[:, active_idx] = v_new


def attention_active(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                     scale: float) -> np.ndarray:
    """[HSA-nl §2.2, items 3-4]: each active query attends to all N cached keys.

    q [B, |A|, H, D], caches [B, N, H, D] (bf16 bits) -> O [B, |A|, H, D] float64.
    O = softmax(q k^T * scale) v per (b, h), evaluated in float64 (READING R8).
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    B, A, H, D = q.shape
    out = np.zeros((B, A, H, D), np.float64)
    if A == 0:
        return out
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * float(scale)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ v[b, :, h, :]
    return out


def qkv_project(x_bits: np.ndarray, w_bits: np.ndarray, bias_bits, heads: int, head_dim: int):
    """[HSA-nl §2.2, items 1-2]: only the active tokens go through the projections; their
    fresh K and V rows are what the cache takes.

    x [B, |A|, Dm], w [3*H*D, Dm] (Q, K, V weights stacked by output row), bias [3*H*D] or
    None, all bf16 bits -> (q, k, v) float64 [B, |A|, H, D]: y = x w^T + bias, evaluated in
    float64 from the bf16 values (no rounding).
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    y = x @ w.T
    if bias_bits is not None:
        y = y + bf16_bits_to_f64(bias_bits)
    B, A = x.shape[0], x.shape[1]
    hd = heads * head_dim
    parts = [y[:, :, p * hd:(p + 1) * hd].reshape(B, A, heads, head_dim) for p in range(3)]
    return parts[0], parts[1], parts[2]


# ----------------------------------------------------------------------------- Euler


def euler_step(x: np.ndarray, v_hat: np.ndarray, v_fresh: np.ndarray, active_idx: np.ndarray,
               sigma_cur, sigma_next):
    """Cached Euler update ([HSA-nl §2.3]).

    The velocity cache takes the fresh velocity of every active token; then every
    token, active or skipped, advances by the same increment (sigma_{i+1} - sigma_i)
    times its cached velocity.  READING R7 for the rounding.  Returns (x, v_hat) new.
    """
    v_hat = np.array(v_hat, dtype=np.float32, copy=True)
    v_hat[active_idx] = v_fresh
    dt = np.float32(np.float32(sigma_next) - np.float32(sigma_cur))
    step = (dt * v_hat).astype(np.float32)
    x = (np.asarray(x, dtype=np.float32) + step).astype(np.float32)
    return x, v_hat


# ----------------------------------------------------------------------------- whole loop


def run_hsa(x0, v_prev, velocity, qkv, prefill, *, T, budgets, group_sizes, m, layers, scale,
            v_cur_for_m0=None, record=None, reselect=False):
    """The full HSA sampling loop, iteration by iteration ([HSA-nl §2.1-§2.4]).

    velocity(i) -> [N, C] float32: the model's velocity prediction at iteration i
        (only the active rows are used).
    qkv(tensor, layer, i, n_rows) -> [B, n_rows, H, D] bf16 bits, tensor in q/k/v:
        the projections of the active tokens, in active_idx order.
    prefill(layer) -> [B, N, H, D] bf16 bits: the cache content before iteration 0.
    record(i, state: dict): optional observer called at the end of every iteration.
    reselect: READING R11, regroup at every all-active iteration after the first selection.

    Returns the final (x, v_hat, group_id, k_caches, v_caches).
    """
    check_budgets(budgets, T)
    x = np.array(x0, dtype=np.float32, copy=True)
    v_hat = np.array(v_prev, dtype=np.float32, copy=True)
    n = x.shape[0]
    g = np.zeros(n, np.int32)
    sig = sigma_schedule(T)
    kc = [np.array(prefill(l), copy=True) for l in range(layers)]
    vc = [np.array(prefill(l), copy=True) for l in range(layers)]
    sel_iter = max(m, 1) - 1
    if m == 0:
        g, _ = select_groups(v_prev, v_cur_for_m0, group_sizes)
    for i in range(T):
        active_idx, active_pos = active_set(g, budgets, T, m, i)
        na = active_idx.shape[0]
        outs = []
        for l in range(layers):
            kv_update(kc[l], vc[l], qkv("k", l, i, na), qkv("v", l, i, na), active_idx)
            outs.append(attention_active(qkv("q", l, i, na), kc[l], vc[l], scale))
        v_fresh = np.asarray(velocity(i), dtype=np.float32)[active_idx]
        r = None
        if (m >= 1 and i == sel_iter) or (reselect and na == n and i >= sel_iter):
            # all tokens are active here, so v_fresh is in token order
            g, r = select_groups(v_hat, v_fresh, group_sizes)
        x, v_hat = euler_step(x, v_hat, v_fresh, active_idx, sig[i], sig[i + 1])
        if record is not None:
            record(i, dict(active_idx=active_idx, active_pos=active_pos, attn=outs,
                           k_caches=[c.copy() for c in kc], v_caches=[c.copy() for c in vc],
                           group_id=g.copy(), score=r, x=x.copy(), v_hat=v_hat.copy(),
                           v_fresh=v_fresh))
    return x, v_hat, g, kc, vc
