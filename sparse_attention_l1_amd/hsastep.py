"""ctypes binding of libhsastep.so (declared in include/hsastep.h).

Argument marshalling only: every function checks the tensors' device, dtype and
contiguity, passes raw pointers plus the current HIP stream, and raises
HsaStepError on a negative status.  All computation happens in the library's
HIP kernels; there is no fallback.  bf16 tensors may be torch.bfloat16 or
torch.uint16/int16 bit patterns.

Importing this module fails loudly if the library has not been built
(``python -m sparse_attention_l1_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhsastep.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m sparse_attention_l1_amd.build`")
lib = ctypes.CDLL(_LIB_PATH)

_p, _i32, _i64, _sz, _f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "hsastep_version": ([], ctypes.c_int),
    "hsastep_error_string": ([ctypes.c_int], ctypes.c_char_p),
    "hsastep_last_error": ([], ctypes.c_char_p),
    "hsastep_workspace_bytes": ([_i64, _i32], _sz),
    "hsastep_n_active": ([_i64, _p, _p, _i32, _i32, _i32, _i32, _p], ctypes.c_int),
    "hsa_select_groups": ([_p, _p, _i64, _i32, _p, _i32, _p, _p, _p, _sz, _p], ctypes.c_int),
    "hsa_active_set": ([_p, _i64, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _sz, _p],
                       ctypes.c_int),
    "hsa_active_set_gather": ([_p, _i64, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _i64,
                               _p, _p, _sz, _p], ctypes.c_int),
    "hsa_active_set_noalloc": ([_p, _i64, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p],
                               ctypes.c_int),
    "hsastep_gather_rows": ([_p, _p, _p, _i64, _i64, _i64, _p], ctypes.c_int),
    "hsa_kv_update": ([_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p], ctypes.c_int),
    "hsa_attention_active": ([_p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _f, _p], ctypes.c_int),
    "hsastep_attention_workspace_bytes": ([_i64, _i64, _i32, _i32, _i32], _sz),
    "hsastep_attention_plan": ([_i64, _i64, _i32, _i32, _i32, _i32, _sz, _p], ctypes.c_int),
    "hsa_attention_active_ws": ([_p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _f, _p, _sz, _p],
                                ctypes.c_int),
    "hsa_euler_step": ([_p, _p, _p, _p, _i64, _i64, _i32, _f, _f, _p], ctypes.c_int),
    "hsa_qkv_project": ([_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p],
                        ctypes.c_int),
    "hsastep_mfma_probe": ([_p, _p, _i32, _i32, _p], ctypes.c_int),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes, _fn.restype = _args, _ret

EXPORTED = tuple(_SIGS)

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4
NOALLOC_MAX_TOKENS = 1 << 24      # HSASTEP_NOALLOC_MAX_TOKENS


class HsaStepError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib.hsastep_last_error().decode() or lib.hsastep_error_string(code).decode()
        super().__init__(f"{where}: {lib.hsastep_error_string(code).decode()} ({code}): {msg}")


def _check(code: int, where: str) -> int:
    if code != OK:
        raise HsaStepError(code, where)
    return code


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_BF16 = (torch.bfloat16, torch.uint16, torch.int16)


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _host_i64(vals: Sequence[int]):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _host_i32(vals: Sequence[int]):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def hsastep_version() -> int:
    return lib.hsastep_version()


def hsastep_workspace_bytes(n_tokens: int, n_groups: int) -> int:
    return int(lib.hsastep_workspace_bytes(n_tokens, n_groups))


def hsastep_n_active(n_tokens: int, budgets: Sequence[int], group_sizes: Sequence[int], T: int,
                     m: int, iteration: int) -> int:
    out = ctypes.c_int64(0)
    _check(lib.hsastep_n_active(n_tokens, _host_i32(budgets), _host_i64(group_sizes),
                                len(budgets), T, m, iteration, ctypes.byref(out)),
           "hsastep_n_active")
    return out.value


def workspace(n_tokens: int, n_groups: int, device="cuda") -> torch.Tensor:
    return torch.empty(hsastep_workspace_bytes(n_tokens, n_groups), dtype=torch.uint8,
                       device=device)


def hsa_select_groups(v_prev: torch.Tensor, v_cur: torch.Tensor, group_sizes: Sequence[int],
                      group_id: torch.Tensor, score: Optional[torch.Tensor],
                      ws: torch.Tensor, stream=None) -> None:
    n, c = v_prev.shape
    if v_cur.shape != v_prev.shape or group_id.shape != (n,):
        raise ValueError("shape mismatch")
    _check(lib.hsa_select_groups(
        _dev(v_prev, "v_prev", (torch.float32,)), _dev(v_cur, "v_cur", (torch.float32,)), n, c,
        _host_i64(group_sizes), len(group_sizes), _dev(group_id, "group_id", (torch.int32,)),
        None if score is None else _dev(score, "score", (torch.float32,)),
        _dev(ws, "workspace", (torch.uint8,)), ws.numel(), _stream(stream)), "hsa_select_groups")


def hsa_active_set(group_id: torch.Tensor, budgets: Sequence[int], group_sizes: Sequence[int],
                   T: int, m: int, iteration: int, active_idx: torch.Tensor,
                   active_pos: torch.Tensor, ws: torch.Tensor, stream=None) -> int:
    n = group_id.shape[0]
    if active_idx.shape != (n,) or active_pos.shape != (n,):
        raise ValueError("active_idx and active_pos must have n_tokens entries")
    out = ctypes.c_int64(0)
    _check(lib.hsa_active_set(
        _dev(group_id, "group_id", (torch.int32,)), n, _host_i32(budgets), _host_i64(group_sizes),
        len(budgets), T, m, iteration, _dev(active_idx, "active_idx", (torch.int32,)),
        _dev(active_pos, "active_pos", (torch.int32,)), ctypes.byref(out),
        _dev(ws, "workspace", (torch.uint8,)), ws.numel(), _stream(stream)), "hsa_active_set")
    return out.value


def hsa_active_set_gather(group_id: torch.Tensor, budgets: Sequence[int],
                          group_sizes: Sequence[int], T: int, m: int, iteration: int,
                          active_idx: torch.Tensor, active_pos: torch.Tensor, rows: torch.Tensor,
                          rows_out: torch.Tensor, ws: torch.Tensor, stream=None) -> int:
    """hsa_active_set plus rows_out[a] = rows[active_idx[a]] for the active tokens (rows and
    rows_out: [n_tokens, ...] with the same row size)."""
    n = group_id.shape[0]
    if active_idx.shape != (n,) or active_pos.shape != (n,):
        raise ValueError("active_idx and active_pos must have n_tokens entries")
    if rows.shape[0] != n or rows_out.shape[0] < n or rows_out.dtype != rows.dtype or \
            rows_out[0].numel() != rows[0].numel():
        raise ValueError("rows and rows_out must hold n_tokens rows of the same size")
    row_bytes = rows[0].numel() * rows.element_size()
    out = ctypes.c_int64(0)
    anyt = (rows.dtype,)
    _check(lib.hsa_active_set_gather(
        _dev(group_id, "group_id", (torch.int32,)), n, _host_i32(budgets), _host_i64(group_sizes),
        len(budgets), T, m, iteration, _dev(active_idx, "active_idx", (torch.int32,)),
        _dev(active_pos, "active_pos", (torch.int32,)), ctypes.byref(out),
        _dev(rows, "rows", anyt), row_bytes, _dev(rows_out, "rows_out", anyt),
        _dev(ws, "workspace", (torch.uint8,)), ws.numel(), _stream(stream)),
        "hsa_active_set_gather")
    return out.value


def hsa_active_set_noalloc(group_id: torch.Tensor, budgets: Sequence[int],
                           group_sizes: Sequence[int], T: int, m: int, iteration: int,
                           active_idx: torch.Tensor, active_pos: torch.Tensor,
                           stream=None) -> int:
    """hsa_active_set with the library's own device scratch in place of a workspace (for
    callers that cannot allocate); calls that overlap on one device race."""
    n = group_id.shape[0]
    if active_idx.shape != (n,) or active_pos.shape != (n,):
        raise ValueError("active_idx and active_pos must have n_tokens entries")
    out = ctypes.c_int64(0)
    _check(lib.hsa_active_set_noalloc(
        _dev(group_id, "group_id", (torch.int32,)), n, _host_i32(budgets), _host_i64(group_sizes),
        len(budgets), T, m, iteration, _dev(active_idx, "active_idx", (torch.int32,)),
        _dev(active_pos, "active_pos", (torch.int32,)), ctypes.byref(out), _stream(stream)),
        "hsa_active_set_noalloc")
    return out.value


def hsastep_gather_rows(dst: torch.Tensor, src: torch.Tensor, index: torch.Tensor, n_rows: int,
                        stream=None) -> None:
    row_bytes = src[0].numel() * src.element_size() if src.dim() > 1 else src.element_size()
    if dst.dtype != src.dtype or dst[0].numel() * dst.element_size() != row_bytes:
        raise ValueError("dst and src rows must match")
    if n_rows > dst.shape[0] or n_rows > index.shape[0]:
        raise ValueError("n_rows exceeds dst or index")
    anyt = (src.dtype,)
    _check(lib.hsastep_gather_rows(_dev(dst, "dst", anyt), _dev(src, "src", anyt),
                                   _dev(index, "index", (torch.int32,)), n_rows, src.shape[0],
                                   row_bytes, _stream(stream)), "hsastep_gather_rows")


def hsa_kv_update(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                  v_new: torch.Tensor, active_idx: torch.Tensor, n_active: int,
                  stream=None) -> None:
    B, N, H, D = k_cache.shape
    if v_cache.shape != k_cache.shape or k_new.shape[0] != B or k_new.shape[2:] != (H, D) or \
            v_new.shape != k_new.shape or k_new.shape[1] < n_active:
        raise ValueError("shape mismatch")
    if n_active > 0 and (k_new.shape[1] != n_active):
        raise ValueError("k_new / v_new must hold exactly n_active rows per batch entry")
    if n_active < 0 or n_active > N or active_idx.numel() < n_active:
        raise ValueError("need 0 <= n_active <= n_tokens and active_idx with >= n_active entries")
    _check(lib.hsa_kv_update(_dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
                             _dev(k_new, "k_new", _BF16), _dev(v_new, "v_new", _BF16),
                             _dev(active_idx, "active_idx", (torch.int32,)), n_active, N, B, H, D,
                             _stream(stream)), "hsa_kv_update")


def hsa_attention_active(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         out: torch.Tensor, softmax_scale: float, stream=None) -> None:
    B, A, H, D = q.shape
    Bk, N, Hk, Dk = k_cache.shape
    if (Bk, Hk, Dk) != (B, H, D) or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch")
    _check(lib.hsa_attention_active(_dev(q, "q", _BF16), _dev(k_cache, "k_cache", _BF16),
                                    _dev(v_cache, "v_cache", _BF16), _dev(out, "out", _BF16), A, N,
                                    B, H, D, float(softmax_scale), _stream(stream)),
           "hsa_attention_active")


def hsastep_attention_workspace_bytes(n_active: int, n_tokens: int, batch: int, heads: int,
                                      head_dim: int) -> int:
    return int(lib.hsastep_attention_workspace_bytes(n_active, n_tokens, batch, heads, head_dim))


def hsastep_attention_plan(n_active: int, n_tokens: int, batch: int, heads: int, head_dim: int,
                           compute_units: int, workspace_bytes: int):
    """(whole tiles, split tiles, key ranges per split tile, keys per range)."""
    out = (ctypes.c_int32 * 4)()
    _check(lib.hsastep_attention_plan(n_active, n_tokens, batch, heads, head_dim, compute_units,
                                      workspace_bytes, out), "hsastep_attention_plan")
    return tuple(out)


def attention_workspace(n_active: int, n_tokens: int, batch: int, heads: int, head_dim: int,
                        device="cuda") -> torch.Tensor:
    n = hsastep_attention_workspace_bytes(n_active, n_tokens, batch, heads, head_dim)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def hsa_attention_active_ws(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            out: torch.Tensor, softmax_scale: float, ws: Optional[torch.Tensor],
                            stream=None) -> None:
    """hsa_attention_active with a workspace (ws=None runs it without one)."""
    B, A, H, D = q.shape
    Bk, N, Hk, Dk = k_cache.shape
    if (Bk, Hk, Dk) != (B, H, D) or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch")
    _check(lib.hsa_attention_active_ws(
        _dev(q, "q", _BF16), _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(out, "out", _BF16), A, N, B, H, D, float(softmax_scale),
        None if ws is None else _dev(ws, "workspace", (torch.uint8,)),
        0 if ws is None else ws.numel(), _stream(stream)), "hsa_attention_active_ws")


def hsa_qkv_project(x_active: torch.Tensor, w_qkv: torch.Tensor, bias: Optional[torch.Tensor],
                    q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    active_idx: torch.Tensor, n_active: int, stream=None) -> None:
    """x_active [B, >= n_active, Dm] bf16 (rows past n_active unused), w_qkv [3*H*D, Dm],
    bias [3*H*D] or None, q_out [B, >= n_active, H, D], caches [B, N, H, D]."""
    B, N, H, D = k_cache.shape
    dm = x_active.shape[-1]
    if v_cache.shape != k_cache.shape or w_qkv.shape != (3 * H * D, dm) or \
            x_active.shape[0] != B or q_out.shape[0] != B or q_out.shape[2:] != (H, D) or \
            (bias is not None and bias.shape != (3 * H * D,)):
        raise ValueError("shape mismatch")
    if n_active < 0 or n_active > N or active_idx.numel() < n_active:
        raise ValueError("need 0 <= n_active <= n_tokens and active_idx with >= n_active entries")
    if x_active.shape[1] < n_active or q_out.shape[1] < n_active:
        raise ValueError("x_active and q_out must hold at least n_active rows")
    if B != 1 and (x_active.shape[1] != n_active or q_out.shape[1] != n_active):
        # rows of batch entry b start at b * n_active, so the row stride must be n_active
        raise ValueError("with batch > 1, x_active and q_out must hold exactly n_active rows")
    _check(lib.hsa_qkv_project(
        _dev(x_active, "x_active", _BF16), _dev(w_qkv, "w_qkv", _BF16),
        None if bias is None else _dev(bias, "bias", _BF16), _dev(q_out, "q_out", _BF16),
        _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(active_idx, "active_idx", (torch.int32,)), n_active, N, B, H, D, dm,
        _stream(stream)), "hsa_qkv_project")


def hsa_euler_step(x: torch.Tensor, v_cache: torch.Tensor, v_fresh: torch.Tensor,
                   active_pos: torch.Tensor, n_active: int, sigma_cur: float, sigma_next: float,
                   stream=None) -> None:
    n, c = x.shape
    if v_cache.shape != x.shape or active_pos.shape != (n,) or v_fresh.shape[1:] != (c,) or \
            v_fresh.shape[0] < n_active:
        raise ValueError("shape mismatch")
    _check(lib.hsa_euler_step(_dev(x, "x", (torch.float32,)),
                              _dev(v_cache, "v_cache", (torch.float32,)),
                              _dev(v_fresh, "v_fresh", (torch.float32,)),
                              _dev(active_pos, "active_pos", (torch.int32,)), n_active, n, c,
                              float(sigma_cur), float(sigma_next), _stream(stream)),
           "hsa_euler_step")


MFMA_PROBE_OPERANDS = 1024 * 8     # bf16 values the probe reads


def hsastep_mfma_probe(operands: torch.Tensor, sink: torch.Tensor, rounds: int,
                       workgroups: int, stream=None) -> float:
    """Launch the sustained-MFMA-rate probe; returns the flops one launch performs."""
    if operands.numel() != MFMA_PROBE_OPERANDS or sink.numel() < workgroups * 256:
        raise ValueError("operands must hold 8192 bf16 values and sink workgroups*256 floats")
    _check(lib.hsastep_mfma_probe(_dev(operands, "operands", _BF16),
                                  _dev(sink, "sink", (torch.float32,)), rounds, workgroups,
                                  _stream(stream)), "hsastep_mfma_probe")
    return float(workgroups) * 4 * 64 * rounds * 32 * 32 * 16 * 2
