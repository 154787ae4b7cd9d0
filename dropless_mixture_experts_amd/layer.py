"""The dropless MoE layer as a sequence of C-ABI calls.

Forward (page "Accelerating dropless MoE training in JAX with NVIDIA
Transformer Engine", Figure 3 paragraph: router -> dispatch -> grouped MLP of
two grouped GEMMs -> combine):
    moe_router_route (bf16; fp32: moe_router_logits -> moe_route) -> moe_permute
      -> moe_grouped_gemm (gate/up, SwiGLU epilogue) -> moe_grouped_gemm (down)
      -> moe_unpermute_combine
    A forward-only layer (no backward buffers) folds the permute into the gate/up
    GEMM's row loads (moe_grouped_gemm_gather) where that form takes the shape, so
    the permuted token matrix is never written.
Backward (routing held fixed):
    moe_permute (gate-scaled dY + d_gates) -> moe_grouped_gemm (KN, SwiGLU backward)
      -> moe_grouped_gemm_wgrad (dW2) -> moe_grouped_gemm (KN, dX_perm)
      -> moe_grouped_gemm_wgrad (dW13) -> moe_unpermute_combine (unit weights, dX)
      [-> moe_route_backward (d_logits) -> moe_router_logits_backward (dWr, dX += router share)]

torch provides device memory and the stream; every arithmetic step runs in
libmoe.so.  Buffers are allocated once per shape and reused, so a forward can
be captured in a HIP graph and replayed.
"""
from __future__ import annotations

import torch

from . import (MOE_EPI_DSWIGLU, MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_LAYOUT_KN, MOE_LAYOUT_NK,
               dtype_code, moe_grouped_gemm, moe_grouped_gemm_gather, moe_grouped_gemm_wgrad,
               moe_grouped_gemm_workspace_size,
               moe_permute, moe_route, moe_route_backward, moe_route_workspace_size,
               moe_router_backward_workspace_size, moe_router_logits, moe_router_logits_backward,
               moe_router_route, moe_router_route_workspace_size, moe_unpermute_combine)


def gather_supported(T: int, d: int, F: int, dtype: torch.dtype) -> bool:
    """Whether moe_grouped_gemm_gather takes the gate/up GEMM of this shape (its header
    states the same bounds: bf16, d % 64 == 0, 32-bit row offsets of x and of the weights)."""
    return (dtype == torch.bfloat16 and d % 64 == 0 and (2 * F) % 16 == 0 and (2 * F + 256) * d * 2 < (1 << 32)
            and T * d * 2 < (1 << 32))


class MoEBuffers:
    """Device buffers of one layer shape.

    ``fuse_permute``: run the gate/up GEMM on gathered token rows instead of a permuted copy
    (None: whenever no backward buffers are asked for and the shape allows it). The backward
    reads the permuted copy, so ``backward=True`` keeps it."""

    def __init__(self, T: int, d: int, E: int, K: int, F: int, dtype: torch.dtype, device="cuda",
                 save_pre: bool = False, backward: bool = False, fuse_permute: bool | None = None):
        self.T, self.d, self.E, self.K, self.F = T, d, E, K, F
        M = T * K
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        act = dict(dtype=dtype, device=dev)
        self.logits = torch.empty((T, E), **f32)
        self.topk_idx = torch.empty((T, K), **i32)
        self.gates = torch.empty((T, K), **f32)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.slot_pos = torch.empty((M,), **i32)
        self.row_src = torch.empty((M,), **i32)
        ws = moe_route_workspace_size(T, E)
        self.ws = torch.empty((max(ws, 256),), dtype=torch.uint8, device=dev)
        self.fused_router = dtype == torch.bfloat16
        if self.fused_router:
            self.rr_ws = torch.empty((max(moe_router_route_workspace_size(T, E), 256),), dtype=torch.uint8,
                                     device=dev)
        # grouped GEMM workspace: zeroed once, every call leaves its counters at zero
        self.gemm_ws = torch.zeros((moe_grouped_gemm_workspace_size(),), dtype=torch.uint8, device=dev)
        if fuse_permute is None:
            fuse_permute = not backward and gather_supported(T, d, F, dtype)
        if fuse_permute and (backward or not gather_supported(T, d, F, dtype)):
            raise ValueError("the permute folds into the gate/up GEMM only for forward-only bf16 layers "
                             "of a shape moe_grouped_gemm_gather takes")
        self.fuse_permute = fuse_permute
        self.x_perm = None if fuse_permute else torch.empty((M, d), **act)
        self.h = torch.empty((M, F), **act)
        self.pre = torch.empty((M, 2 * F), **act) if (save_pre or backward) else None
        self.y_perm = torch.empty((M, d), **act)
        self.y = torch.empty((T, d), **act)
        if backward:
            self.dy_perm = torch.empty((M, d), **act)
            self.d_gates = torch.empty((T, K), **f32)
            self.d_pre = torch.empty((M, 2 * F), **act)
            self.dx_perm = torch.empty((M, d), **act)
            self.dx = torch.empty((T, d), **act)
            self.dw13 = torch.empty((E, 2 * F, d), **f32)
            self.dw2 = torch.empty((E, d, F), **f32)
            self.d_logits = torch.empty((T, E), **f32)
            self.dw_router = torch.empty((E, d), **f32)
            code = dtype_code(torch.empty(0, dtype=dtype))
            self.rb_ws = torch.empty((max(moe_router_backward_workspace_size(T, d, E, code), 256),),
                                     dtype=torch.uint8, device=dev)


def forward_steps(x, w_router, bias, w13, w2, K: int, score: int, renorm: bool, bufs: MoEBuffers, logits=None,
                  stream=None):
    """The forward as (name, call) pairs in launch order: one C-ABI call each.

    ``logits`` (fp32 [T, E]) skips the router product and routes on the given values."""
    b = bufs
    steps = []
    if logits is None and b.fused_router:
        # product and routing in one call; the logits are still written for the router backward
        steps.append(("router_route", lambda: moe_router_route(
            x, w_router, bias, K, score, renorm, b.logits, b.topk_idx, b.gates, b.counts, b.offsets, b.slot_pos,
            b.row_src, b.rr_ws, stream=stream)))
    else:
        if logits is None:
            steps.append(("router", lambda: moe_router_logits(x, w_router, b.logits, stream=stream)))
            logits = b.logits
        steps.append(("route", lambda: moe_route(logits, bias, K, score, renorm, b.topk_idx, b.gates, b.counts,
                                                 b.offsets, b.slot_pos, b.row_src, b.ws, stream=stream)))
    if b.fuse_permute:
        steps.append(("gemm_gate_up", lambda: moe_grouped_gemm_gather(
            x, b.row_src, K, w13, b.offsets, b.h, MOE_EPI_SWIGLU, epi_save=b.pre, workspace=b.gemm_ws,
            stream=stream)))
    else:
        steps += [
            ("permute", lambda: moe_permute(x, K, b.slot_pos, b.x_perm, stream=stream)),
            ("gemm_gate_up", lambda: moe_grouped_gemm(b.x_perm, w13, MOE_LAYOUT_NK, b.offsets, b.h, MOE_EPI_SWIGLU,
                                                      epi_save=b.pre, workspace=b.gemm_ws, stream=stream)),
        ]
    steps += [
        ("gemm_down", lambda: moe_grouped_gemm(b.h, w2, MOE_LAYOUT_NK, b.offsets, b.y_perm, MOE_EPI_NONE,
                                               workspace=b.gemm_ws, stream=stream)),
        ("combine", lambda: moe_unpermute_combine(b.y_perm, b.slot_pos, b.gates, b.T, K, b.y, stream=stream)),
    ]
    return steps


def layer_forward(x, w_router, bias, w13, w2, K: int, score: int, renorm: bool, bufs: MoEBuffers,
                  logits=None, stream=None):
    """y = combine(down(SwiGLU(gate_up(permute(x))))) with top-K routing; returns bufs.y.

    ``logits`` (fp32 [T, E]) skips the router product and routes on the given values."""
    for _, call in forward_steps(x, w_router, bias, w13, w2, K, score, renorm, bufs, logits, stream):
        call()
    return bufs.y


def backward_steps(dy, w13, w2, K: int, bufs: MoEBuffers, stream=None, router=None):
    """The backward as (name, call) pairs in launch order (routing of the last forward held fixed)."""
    b = bufs
    steps = [
        ("combine_bwd", lambda: moe_permute(dy, K, b.slot_pos, b.dy_perm, row_scale=b.gates, y_perm_dot=b.y_perm,
                                            dgate_out=b.d_gates, stream=stream)),
        ("dgrad_down_dswiglu", lambda: moe_grouped_gemm(b.dy_perm, w2, MOE_LAYOUT_KN, b.offsets, b.d_pre,
                                                        MOE_EPI_DSWIGLU, epi_in=b.pre, workspace=b.gemm_ws,
                                                        stream=stream)),
        ("wgrad_down", lambda: moe_grouped_gemm_wgrad(b.h, b.dy_perm, b.offsets, b.dw2, stream=stream)),
        ("dgrad_gate_up", lambda: moe_grouped_gemm(b.d_pre, w13, MOE_LAYOUT_KN, b.offsets, b.dx_perm, MOE_EPI_NONE,
                                                   workspace=b.gemm_ws, stream=stream)),
        ("wgrad_gate_up", lambda: moe_grouped_gemm_wgrad(b.x_perm, b.d_pre, b.offsets, b.dw13, stream=stream)),
        ("permute_bwd", lambda: moe_unpermute_combine(b.dx_perm, b.slot_pos, None, b.T, K, b.dx, stream=stream)),
    ]
    if router is not None:
        steps += [
            ("route_bwd", lambda: moe_route_backward(router["logits"], router.get("bias"), b.topk_idx, b.d_gates,
                                                     router["score"], router["renorm"], b.d_logits, stream=stream)),
            ("router_bwd", lambda: moe_router_logits_backward(b.d_logits, router["x"], router["w_router"],
                                                              b.dw_router, b.dx, b.rb_ws, accumulate=True,
                                                              stream=stream)),
        ]
    return steps


def layer_backward(dy, w13, w2, K: int, bufs: MoEBuffers, stream=None, router=None):
    """Gradients of <dY, Y> with the routing of the last forward held fixed.

    Returns (dx, dw13, dw2, d_gates) in bufs.  With ``router`` = dict(logits, x, w_router,
    bias, score, renorm) of that forward, also takes d_gates back through the gates (top-K
    held fixed) to bufs.d_logits and bufs.dw_router, and adds the router's share to dx."""
    for _, call in backward_steps(dy, w13, w2, K, bufs, stream, router):
        call()
    return bufs.dx, bufs.dw13, bufs.dw2, bufs.d_gates
