"""The DiT-MoE sparse MoE feed-forward layer as one sequence of C-ABI calls.

    gate -> permute -> routed expert MLPs -> shared expert MLPs -> combine
         -> balance statistic

("Scaling Diffusion Transformers to 16 Billion Parameters", Methods: eq.
MoE(x), eq. MLP(x), shared expert routing, eq. L_balance; "DiT-MoE" hub
page, section 1: the softmax top-k gate; "Expert Race" abstract for the race
routing.)

This module holds device weights and preallocated buffers and issues the
calls in order on the current stream.  Every step runs in libmoe.so; torch
only provides device memory and the stream.  Nothing here synchronises.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib, ops

ROUTES = {"topk": _lib.MOE_ROUTE_TOPK, "race": _lib.MOE_ROUTE_EXPERT_RACE}
BALANCE = {"sequence": _lib.MOE_BAL_PER_SEQUENCE, "global": _lib.MOE_BAL_GLOBAL}


def _to_device(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    """Upload an fp32 array holding exact bf16 (or fp32) values."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == torch.bfloat16:
        # exact: the values are bf16-representable
        t = t.to(torch.bfloat16)
    return t.to(device)


@dataclass
class LayerWeights:
    """Device weights of one layer (layouts of include/moe.h)."""
    w_gate: torch.Tensor            # [E][D] fp32
    bias: Optional[torch.Tensor]    # [E] fp32 or None
    w1: torch.Tensor                # [E][H][D]
    w2: torch.Tensor                # [E][D][H]
    w1s: Optional[torch.Tensor]     # [1][n_s*H][D]  shared experts stacked
    w2s: Optional[torch.Tensor]     # [1][D][n_s*H]

    @staticmethod
    def from_inputs(inp, device="cuda") -> "LayerWeights":
        cfg = inp.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        w1s = w2s = None
        if cfg.n_s > 0:
            # n_s MLPs summed with weight 1 == one MLP of hidden n_s*H: W1 rows
            # and W2 columns concatenated.
            w1s = _to_device(inp.w1s.reshape(1, cfg.n_s * cfg.H, cfg.D), dt, device)
            w2s = _to_device(np.transpose(inp.w2s, (1, 0, 2)).reshape(
                1, cfg.D, cfg.n_s * cfg.H), dt, device)
        return LayerWeights(
            w_gate=_to_device(inp.w_gate, torch.float32, device),
            bias=None if inp.bias is None else _to_device(inp.bias, torch.float32,
                                                           device),
            w1=_to_device(inp.w1, dt, device),
            w2=_to_device(inp.w2, dt, device),
            w1s=w1s, w2s=w2s)


class LayerBuffers:
    """Every intermediate and output tensor of one forward pass, allocated
    once for a fixed token count.  With save_u (training, bf16 layers) the
    expert MLPs' pre-activations are kept too, so that the backward pass
    does not recompute them."""

    def __init__(self, cfg, device="cuda", gather: bool = False,
                 y_rows_f32: bool = False, save_u: bool = False):
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        N, D, H, E, K, n_s = cfg.N, cfg.D, cfg.H, cfg.E, cfg.K, cfg.n_s
        Kmax, A = cfg.Kmax, cfg.A
        route = ROUTES[cfg.route]
        f32, i32, i64 = torch.float32, torch.int32, torch.int64
        dev = device
        self.gather = gather
        self.probs = torch.empty(N, E, dtype=f32, device=dev)
        self.topk_idx = torch.empty(N, Kmax, dtype=i32, device=dev)
        self.topk_w = torch.empty(N, Kmax, dtype=f32, device=dev)
        gws = ops.gate_workspace_size(N, E, K, route)
        self.gate_ws = torch.empty(max(gws, 1), dtype=torch.uint8, device=dev)
        self.expert_counts = torch.empty(E, dtype=i32, device=dev)
        self.expert_offsets = torch.empty(E + 1, dtype=i64, device=dev)
        self.row_token = torch.empty(max(A, 1), dtype=i32, device=dev)
        self.slot_row = torch.empty(N, Kmax, dtype=i32, device=dev)
        self.x_perm = None if gather else torch.empty(A, D, dtype=dt, device=dev)
        pws = ops.permute_workspace_size(N, E, Kmax)
        self.perm_ws = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
        self.h = torch.empty(A, H, dtype=dt, device=dev)
        if save_u and dt != torch.bfloat16:
            raise ValueError("saved pre-activations need a bf16 layer")
        self.u = torch.empty(A, H, dtype=dt, device=dev) if save_u else None
        ydt = f32 if (y_rows_f32 or dt == f32) else dt
        self.y_rows = torch.empty(A, D, dtype=ydt, device=dev)
        if n_s > 0:
            self.shared_offsets = torch.tensor([0, N], dtype=i64, device=dev)
            self.h_shared = torch.empty(N, n_s * H, dtype=dt, device=dev)
            self.u_shared = (torch.empty(N, n_s * H, dtype=dt, device=dev)
                             if save_u else None)
            self.y_shared = torch.empty(N, D, dtype=dt, device=dev)
        else:
            self.shared_offsets = self.h_shared = self.y_shared = None
            self.u_shared = None
        self.y = torch.empty(N, D, dtype=dt, device=dev)
        # the routed experts' stage 2 splits its last round of tiles along k
        # into this workspace (bf16 layers)
        self.split_ws = (torch.empty(ops.ffn_split_workspace_size(),
                                     dtype=torch.uint8, device=dev)
                         if cfg.dtype == "bf16" else None)
        self.gate_bal_ws = self.route_ws = None
        if route == ROUTES["topk"]:
            bws = ops.gate_balance_workspace_size(cfg.B, cfg.T, E)
            self.gate_bal_ws = torch.empty(max(bws, 1), dtype=torch.uint8,
                                           device=dev)
            rws = ops.gate_route_workspace_size(cfg.B, cfg.T, E)
            self.route_ws = torch.empty(max(rws, 1), dtype=torch.uint8,
                                        device=dev)
        self.bal_counts = torch.empty(cfg.B, E, dtype=i32, device=dev)
        self.bal_psum = torch.empty(cfg.B, E, dtype=f32, device=dev)
        self.loss = torch.empty(1, dtype=f32, device=dev)


def gate(cfg, x, wts: LayerWeights, buf: LayerBuffers):
    ops.moe_gate_topk(x, wts.w_gate, wts.bias, cfg.K, ROUTES[cfg.route],
                      buf.probs, buf.topk_idx, buf.topk_w, buf.gate_ws)


def fuses_balance(cfg) -> bool:
    """Top-K layers compute the balance statistic in the gate's call (its
    kernel reduces each 16-token group where the shape allows)."""
    return cfg.route == "topk"


def gate_balance(cfg, x, wts: LayerWeights, buf: LayerBuffers,
                 mode: str = "sequence"):
    ops.moe_gate_topk_balance(x, wts.w_gate, wts.bias, cfg.B, cfg.T, cfg.K,
                              cfg.alpha, BALANCE[mode], buf.probs,
                              buf.topk_idx, buf.topk_w, buf.bal_counts,
                              buf.bal_psum, buf.loss, buf.gate_bal_ws)


def fuses_route(cfg, buf: LayerBuffers) -> bool:
    """Top-K layers whose routed rows are gathered in the GEMM (no x_perm)
    route in one call: the gate, the balance statistic and the permutation's
    index tensors."""
    return fuses_balance(cfg) and buf.gather


def gate_route(cfg, x, wts: LayerWeights, buf: LayerBuffers,
               mode: str = "sequence"):
    ops.moe_gate_route(x, wts.w_gate, wts.bias, cfg.B, cfg.T, cfg.K,
                       cfg.alpha, BALANCE[mode], buf.probs, buf.topk_idx,
                       buf.topk_w, buf.bal_counts, buf.bal_psum, buf.loss,
                       buf.expert_counts, buf.expert_offsets, buf.row_token,
                       buf.slot_row, buf.route_ws)


def permute(cfg, x, buf: LayerBuffers):
    ops.moe_permute(x, buf.topk_idx, cfg.E, cfg.K, buf.expert_counts,
                    buf.expert_offsets, buf.row_token, buf.slot_row, buf.x_perm,
                    buf.perm_ws)


def routed_ffn(cfg, x, wts: LayerWeights, buf: LayerBuffers,
               stages: int = _lib.MOE_FFN_BOTH):
    if buf.gather:
        ops.moe_grouped_ffn(x, buf.row_token, cfg.A, buf.expert_offsets, wts.w1,
                            None, wts.w2, None, buf.h, buf.y_rows, stages,
                            buf.u, buf.split_ws)
    else:
        ops.moe_grouped_ffn(buf.x_perm, None, cfg.A, buf.expert_offsets, wts.w1,
                            None, wts.w2, None, buf.h, buf.y_rows, stages,
                            buf.u, buf.split_ws)


def shared_ffn(cfg, x, wts: LayerWeights, buf: LayerBuffers,
               stages: int = _lib.MOE_FFN_BOTH):
    if cfg.n_s > 0:
        ops.moe_grouped_ffn(x, None, cfg.N, buf.shared_offsets, wts.w1s, None,
                            wts.w2s, None, buf.h_shared, buf.y_shared, stages,
                            buf.u_shared)


def fuses_combine(cfg, buf: LayerBuffers) -> bool:
    """The shared experts' stage 2 and the combine run as one kernel for
    bf16 layers with shared experts, bf16 routed outputs and at most 16
    slots per token (top-K routing, or Expert Race with E <= 16)."""
    return (cfg.dtype == "bf16" and cfg.n_s > 0 and cfg.Kmax <= 16
            and buf.y_rows.dtype == torch.bfloat16)


def shared_down_combine(cfg, wts: LayerWeights, buf: LayerBuffers):
    """Stage 2 of the shared experts fused with the weighted combine: y."""
    ops.moe_ffn_down_combine(buf.h_shared, wts.w2s, None, buf.y_rows,
                             buf.slot_row, buf.topk_w, buf.y)


def combine(cfg, buf: LayerBuffers):
    ops.moe_combine(buf.y_rows, buf.slot_row, buf.topk_w, buf.y_shared, buf.y)


def balance(cfg, buf: LayerBuffers, mode: str = "sequence"):
    ops.moe_balance_stats(buf.probs, buf.topk_idx, cfg.B, cfg.T, cfg.K,
                          cfg.alpha, BALANCE[mode], buf.bal_counts,
                          buf.bal_psum, buf.loss)


# The layer as a list of single-kernel-group calls, in order (the expert
# MLPs split into their two GEMM stages): the same work as forward().  Both
# up-projections run before both down-projections: the shared one then reads
# x while the gate's and the routed stage's reads of it still sit in the
# 256 MB memory-side cache, instead of after 604 MB of h have streamed
# through it (measured: 2% less time per layer than routed MLP, then shared).
UP, DOWN = _lib.MOE_FFN_UP, _lib.MOE_FFN_DOWN
STEPS = (("gate", lambda c, x, w, b: gate(c, x, w, b)),
         ("permute", lambda c, x, w, b: permute(c, x, b)),
         ("routed_up", lambda c, x, w, b: routed_ffn(c, x, w, b, UP)),
         ("shared_up", lambda c, x, w, b: shared_ffn(c, x, w, b, UP)),
         ("routed_down", lambda c, x, w, b: routed_ffn(c, x, w, b, DOWN)),
         ("shared_down", lambda c, x, w, b: shared_ffn(c, x, w, b, DOWN)),
         ("combine", lambda c, x, w, b: combine(c, b)),
         ("balance", lambda c, x, w, b: balance(c, b)))

# The fused calls forward() makes instead: the gate with the balance
# statistic (top-K routing) and, when the routed rows are gathered in the
# GEMM, also with the permutation; and the shared experts' stage 2 with the
# combine (when fuses_combine(cfg, buf)): y bit for bit the same either way.
GATE_BALANCE_STEP = ("gate_balance",
                     lambda c, x, w, b: gate_balance(c, x, w, b))
GATE_ROUTE_STEP = ("gate_route", lambda c, x, w, b: gate_route(c, x, w, b))
DOWN_COMBINE_STEP = ("shared_down_combine",
                     lambda c, x, w, b: shared_down_combine(c, w, b))


def steps(cfg, buf: LayerBuffers):
    """The calls forward() makes for this layer, in order."""
    out = []
    for s in STEPS:
        name = s[0]
        if cfg.n_s == 0 and name.startswith("shared"):
            continue
        if fuses_balance(cfg) and name == "balance":
            continue
        if fuses_route(cfg, buf) and name == "permute":
            continue
        if fuses_combine(cfg, buf) and name == "combine":
            continue
        if fuses_route(cfg, buf) and name == "gate":
            s = GATE_ROUTE_STEP
        elif fuses_balance(cfg) and name == "gate":
            s = GATE_BALANCE_STEP
        elif fuses_combine(cfg, buf) and name == "shared_down":
            s = DOWN_COMBINE_STEP
        out.append(s)
    return tuple(out)


def forward(cfg, x: torch.Tensor, wts: LayerWeights, buf: LayerBuffers,
            balance_mode: str = "sequence") -> LayerBuffers:
    """One pass of the whole layer; results land in ``buf``."""
    if fuses_route(cfg, buf):
        gate_route(cfg, x, wts, buf, balance_mode)
    else:
        if fuses_balance(cfg):
            gate_balance(cfg, x, wts, buf, balance_mode)
        else:
            gate(cfg, x, wts, buf)
        permute(cfg, x, buf)
    routed_ffn(cfg, x, wts, buf, UP)
    shared_ffn(cfg, x, wts, buf, UP)
    routed_ffn(cfg, x, wts, buf, DOWN)
    if fuses_combine(cfg, buf):
        shared_down_combine(cfg, wts, buf)
    else:
        shared_ffn(cfg, x, wts, buf, DOWN)
        combine(cfg, buf)
    if not fuses_balance(cfg):
        balance(cfg, buf, balance_mode)
    return buf


# ---------------------------------------------------------------- backward --

class BackwardBuffers:
    """Gradients and workspaces of one backward pass (bf16 layers)."""

    def __init__(self, cfg, device="cuda"):
        if cfg.dtype != "bf16":
            raise ValueError("the backward pass takes bf16 layers")
        dt, f32, i32 = torch.bfloat16, torch.float32, torch.int32
        N, D, H, E, Kmax, A, n_s = cfg.N, cfg.D, cfg.H, cfg.E, cfg.Kmax, cfg.A, cfg.n_s
        dev = device
        self.dy_rows = torch.empty(A, D, dtype=dt, device=dev)
        self.slot_grad = torch.empty(N, Kmax, dtype=f32, device=dev)
        self.dx_rows = torch.empty(A, D, dtype=dt, device=dev)
        self.dw1 = torch.empty(E, H, D, dtype=f32, device=dev)
        self.dw2 = torch.empty(E, D, H, dtype=f32, device=dev)
        ws = ops.ffn_backward_workspace_size(A, E, D, H)
        if n_s > 0:
            self.dx_shared = torch.empty(N, D, dtype=dt, device=dev)
            self.dw1s = torch.empty(1, n_s * H, D, dtype=f32, device=dev)
            self.dw2s = torch.empty(1, D, n_s * H, dtype=f32, device=dev)
            ws = max(ws, ops.ffn_backward_workspace_size(N, 1, D, n_s * H))
        else:
            self.dx_shared = self.dw1s = self.dw2s = None
        self.ffn_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.dx = torch.empty(N, D, dtype=dt, device=dev)
        self.dw_gate = torch.empty(E, D, dtype=f32, device=dev)
        self.dbias = torch.empty(E, dtype=f32, device=dev)
        gws = ops.gate_backward_workspace_size(N, E, D)
        self.gate_ws = torch.empty(max(gws, 1), dtype=torch.uint8, device=dev)


def combine_backward(cfg, buf, grads, dy):
    ops.moe_combine_backward(dy, buf.y_rows, buf.slot_row, buf.topk_w,
                             grads.dy_rows, grads.slot_grad)


def routed_ffn_backward(cfg, x, wts, buf, grads):
    x_rows, row_index = (x, buf.row_token) if buf.gather else (buf.x_perm, None)
    saved = buf.u is not None
    ops.moe_grouped_ffn_backward(x_rows, row_index, cfg.A, buf.expert_offsets,
                                 wts.w1, None, wts.w2, grads.dy_rows,
                                 grads.ffn_ws, grads.dx_rows, grads.dw1,
                                 grads.dw2, buf.u, buf.h if saved else None)


def shared_ffn_backward(cfg, x, wts, buf, grads, dy):
    if cfg.n_s > 0:
        saved = buf.u_shared is not None
        ops.moe_grouped_ffn_backward(x, None, cfg.N, buf.shared_offsets,
                                     wts.w1s, None, wts.w2s, dy, grads.ffn_ws,
                                     grads.dx_shared, grads.dw1s, grads.dw2s,
                                     buf.u_shared,
                                     buf.h_shared if saved else None)


def gate_backward(cfg, x, wts, buf, grads, dloss, balance_mode="sequence"):
    ops.moe_gate_backward(x, wts.w_gate, buf.probs, buf.topk_idx,
                          grads.slot_grad, buf.bal_counts, cfg.B, cfg.T,
                          cfg.K, cfg.alpha, dloss, BALANCE[balance_mode],
                          grads.dx_rows, buf.slot_row, grads.dx_shared,
                          grads.dx, grads.dw_gate, grads.dbias, grads.gate_ws)


# The backward pass as named calls, in order (same work as backward()):
# each takes (cfg, x, weights, forward buffers, gradients, dy, dloss).
BACKWARD_STEPS = (
    ("combine_backward", lambda c, x, w, b, g, dy, dl: combine_backward(c, b, g, dy)),
    ("routed_ffn_backward", lambda c, x, w, b, g, dy, dl: routed_ffn_backward(c, x, w, b, g)),
    ("shared_ffn_backward", lambda c, x, w, b, g, dy, dl: shared_ffn_backward(c, x, w, b, g, dy)),
    ("gate_backward", lambda c, x, w, b, g, dy, dl: gate_backward(c, x, w, b, g, dl)),
)


def backward(cfg, x, wts: LayerWeights, buf: LayerBuffers,
             grads: BackwardBuffers, dy: torch.Tensor, dloss: float = 1.0,
             balance_mode: str = "sequence") -> BackwardBuffers:
    """Gradients of <dy, y> + dloss * L_balance after forward() (same
    buffers and balance mode): combine, routed experts, shared experts, gate
    and dx.  Buffers made with save_u give the expert MLPs the forward's
    pre-activations and activations (no recomputation)."""
    combine_backward(cfg, buf, grads, dy)
    routed_ffn_backward(cfg, x, wts, buf, grads)
    shared_ffn_backward(cfg, x, wts, buf, grads, dy)
    gate_backward(cfg, x, wts, buf, grads, dloss, balance_mode)
    return grads
