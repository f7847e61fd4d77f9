"""Tensor-level binding of the five C-ABI calls, same names as include/moe.h.

Argument marshalling only: tensors become device pointers, dtypes become
moe_dtype codes, and every call is enqueued on torch's current HIP stream.
Outputs are caller-provided tensors (allocate them once and reuse them).
All arithmetic happens in libmoe.so.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}


def dtype_code(t: torch.dtype) -> int:
    try:
        return _DT[t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t}") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _src_rows(x_rows) -> int:
    """Row count of a matrix the expert MLPs gather rows from."""
    return 0 if x_rows is None else int(x_rows.shape[0])


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def gate_workspace_size(N: int, E: int, K: int, route: int) -> int:
    return _lib.load().moe_gate_workspace_size(N, E, K, route)


def permute_workspace_size(N: int, E: int, Kmax: int) -> int:
    return _lib.load().moe_permute_workspace_size(N, E, Kmax)


def moe_gate_topk(x, w_gate, logit_bias, K: int, route: int, probs, topk_idx,
                  topk_w, workspace=None):
    N, D = x.shape
    E = w_gate.shape[0]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.call("moe_gate_topk", _ptr(x), dtype_code(x.dtype), _ptr(w_gate),
              _ptr(logit_bias), N, D, E, K, route, _ptr(probs), _ptr(topk_idx),
              _ptr(topk_w), _ptr(workspace), ws, _stream())


def moe_permute(x, topk_idx, E: int, K: int, expert_counts, expert_offsets,
                row_token, slot_row, x_perm, workspace):
    N, D = x.shape
    Kmax = topk_idx.shape[1]
    ws = workspace.numel() * workspace.element_size()
    _lib.call("moe_permute", _ptr(x), dtype_code(x.dtype), _ptr(topk_idx), N,
              D, E, Kmax, K, _ptr(expert_counts), _ptr(expert_offsets),
              _ptr(row_token), _ptr(slot_row), _ptr(x_perm), _ptr(workspace),
              ws, _stream())


def moe_permute_noalloc(x, topk_idx, E: int, K: int, expert_counts,
                        expert_offsets, row_token, slot_row, x_perm):
    """moe_permute on the library's static scratch (no workspace)."""
    N, D = x.shape
    Kmax = topk_idx.shape[1]
    _lib.call("moe_permute_noalloc", _ptr(x), dtype_code(x.dtype),
              _ptr(topk_idx), N, D, E, Kmax, K, _ptr(expert_counts),
              _ptr(expert_offsets), _ptr(row_token), _ptr(slot_row),
              _ptr(x_perm), _stream())


def ffn_split_workspace_size() -> int:
    return _lib.load().moe_grouped_ffn_split_workspace_size()


def moe_grouped_ffn(x_rows, row_index, total_rows: int, group_offsets, w1, b1,
                    w2, b2, h_ws, y_rows, stages: int = _lib.MOE_FFN_BOTH,
                    u_ws=None, split_ws=None):
    """moe_grouped_ffn, or with split_ws (a uint8 tensor of at least
    ffn_split_workspace_size() bytes) moe_grouped_ffn_split."""
    if w1 is not None:
        G, H, D = w1.shape
    else:                      # stage 2 alone
        G, D, H = w2.shape
    args = [_ptr(x_rows), _ptr(row_index), _src_rows(x_rows),
            dtype_code(h_ws.dtype), total_rows, _ptr(group_offsets), G, D, H,
            _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(h_ws), _ptr(u_ws),
            _ptr(y_rows),
            dtype_code(y_rows.dtype if y_rows is not None else h_ws.dtype),
            stages]
    if split_ws is None:
        _lib.call("moe_grouped_ffn", *args, _stream())
    else:
        _lib.call("moe_grouped_ffn_split", *args, _ptr(split_ws),
                  split_ws.numel() * split_ws.element_size(), _stream())


def moe_grouped_mlp_fused(x_rows, row_index, total_rows: int, group_offsets,
                          w1, b1, w2, b2, y_rows):
    G, H, D = w1.shape
    _lib.call("moe_grouped_mlp_fused", _ptr(x_rows), _ptr(row_index),
              _src_rows(x_rows), dtype_code(w1.dtype), total_rows, _ptr(group_offsets), G, D, H,
              _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(y_rows),
              dtype_code(y_rows.dtype), _stream())


def moe_combine(y_rows, slot_row, topk_w, y_shared, y):
    N, D = y.shape
    Kmax = slot_row.shape[1]
    sh = _lib.MOE_F32 if y_shared is None else dtype_code(y_shared.dtype)
    _lib.call("moe_combine", _ptr(y_rows), dtype_code(y_rows.dtype),
              _ptr(slot_row), _ptr(topk_w), N, D, Kmax, _ptr(y_shared), sh,
              _ptr(y), dtype_code(y.dtype), _stream())


def moe_balance_stats(probs, topk_idx, B: int, T: int, K: int, alpha: float,
                      mode: int, counts, prob_sums, loss):
    E = probs.shape[1]
    Kmax = topk_idx.shape[1]
    _lib.call("moe_balance_stats", _ptr(probs), _ptr(topk_idx), B, T, E, Kmax,
              K, alpha, mode, _ptr(counts), _ptr(prob_sums), _ptr(loss),
              _stream())


def gate_balance_workspace_size(B: int, T: int, E: int) -> int:
    return _lib.load().moe_gate_balance_workspace_size(B, T, E)


def moe_gate_topk_balance(x, w_gate, logit_bias, B: int, T: int, K: int,
                          alpha: float, mode: int, probs, topk_idx, topk_w,
                          counts, prob_sums, loss, workspace):
    N, D = x.shape
    if N != B * T:
        raise ValueError(f"x has {N} rows, expected B*T = {B * T}")
    E = w_gate.shape[0]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.call("moe_gate_topk_balance", _ptr(x), dtype_code(x.dtype),
              _ptr(w_gate), _ptr(logit_bias), B, T, D, E, K, alpha, mode,
              _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
              _ptr(prob_sums), _ptr(loss), _ptr(workspace), ws, _stream())


def gate_route_workspace_size(B: int, T: int, E: int) -> int:
    return _lib.load().moe_gate_route_workspace_size(B, T, E)


def moe_gate_route(x, w_gate, logit_bias, B: int, T: int, K: int,
                   alpha: float, mode: int, probs, topk_idx, topk_w, counts,
                   prob_sums, loss, expert_counts, expert_offsets, row_token,
                   slot_row, workspace):
    N, D = x.shape
    if N != B * T:
        raise ValueError(f"x has {N} rows, expected B*T = {B * T}")
    E = w_gate.shape[0]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.call("moe_gate_route", _ptr(x), dtype_code(x.dtype), _ptr(w_gate),
              _ptr(logit_bias), B, T, D, E, K, alpha, mode, _ptr(probs),
              _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(prob_sums),
              _ptr(loss), _ptr(expert_counts), _ptr(expert_offsets),
              _ptr(row_token), _ptr(slot_row), _ptr(workspace), ws, _stream())


def moe_routing_histogram(topk_idx, B: int, T: int, E: int, pos_counts,
                          image_tag=None, tag_counts=None):
    """Add one batch's expert-selection counts by position (and by image
    tag) into the int64 totals pos_counts [T][E] (and tag_counts)."""
    Kmax = topk_idx.shape[1]
    n_tags = 0 if tag_counts is None else tag_counts.shape[0]
    _lib.call("moe_routing_histogram", _ptr(topk_idx), B, T, E, Kmax,
              _ptr(image_tag), n_tags, _ptr(pos_counts), _ptr(tag_counts),
              _stream())


def moe_ffn_down_combine(h, w2, b2, y_rows, slot_row, topk_w, y):
    """Shared experts' stage 2 fused with the weighted combine: y [N][D]."""
    N, H = h.shape
    D = w2.shape[-2]
    _lib.call("moe_ffn_down_combine", _ptr(h), dtype_code(h.dtype), N, D, H,
              _ptr(w2), _ptr(b2), _ptr(y_rows), _ptr(slot_row), _ptr(topk_w),
              slot_row.shape[1], _ptr(y), _stream())


# ---------------------------------------------------------------- backward --

def moe_combine_backward(dy, y_rows, slot_row, topk_w, dy_rows, slot_grad):
    N, D = dy.shape
    _lib.call("moe_combine_backward", _ptr(dy), dtype_code(dy.dtype),
              _ptr(y_rows), dtype_code(y_rows.dtype), _ptr(slot_row),
              _ptr(topk_w), N, D, slot_row.shape[1], _ptr(dy_rows),
              _ptr(slot_grad), _stream())


def ffn_backward_workspace_size(total_rows: int, G: int, D: int, H: int) -> int:
    return int(_lib.load().moe_ffn_backward_workspace_size(total_rows, G, D, H))


def moe_grouped_ffn_backward(x_rows, row_index, total_rows: int, group_offsets,
                             w1, b1, w2, dy_rows, workspace, dx_rows, dw1, dw2,
                             u_rows=None, h_rows=None):
    G, H, D = w1.shape
    _lib.call("moe_grouped_ffn_backward", _ptr(x_rows), _ptr(row_index),
              _src_rows(x_rows), dtype_code(w1.dtype), total_rows, _ptr(group_offsets), G, D, H,
              _ptr(w1), _ptr(b1), _ptr(w2), _ptr(dy_rows), _ptr(u_rows),
              _ptr(h_rows), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _ptr(dx_rows),
              dtype_code(dx_rows.dtype), _ptr(dw1), _ptr(dw2), _stream())


def gate_backward_workspace_size(N: int, E: int, D: int) -> int:
    return int(_lib.load().moe_gate_backward_workspace_size(N, E, D))


def moe_gate_backward(x, w_gate, probs, topk_idx, slot_grad, counts, B: int,
                      T: int, K: int, alpha: float, dloss: float, mode: int,
                      dx_rows, slot_row, dx_shared, dx, dw_gate, dbias,
                      workspace):
    E, D = w_gate.shape
    _lib.call("moe_gate_backward", _ptr(x), dtype_code(x.dtype), _ptr(w_gate),
              _ptr(probs), _ptr(topk_idx), _ptr(slot_grad), _ptr(counts), B, T,
              D, E, topk_idx.shape[1], K, alpha, dloss, mode, _ptr(dx_rows),
              _ptr(slot_row), _ptr(dx_shared), dtype_code(dx.dtype), _ptr(dx),
              _ptr(dw_gate), _ptr(dbias), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream())
