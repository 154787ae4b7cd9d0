"""Dropless MoE layer hot path for AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libmoe.so`` (declared in ``include/moe.h``).  Each
function has the name of the C entry point it calls and only marshals
arguments: torch tensors are passed as device pointers and the current HIP
stream as ``moe_stream_t``.  Every step of the layer runs in the library's HIP
kernels; there is no other code path.  Importing the package does not load the
library; the first call does, and raises if ``libmoe.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_HIP_ERROR, MOE_SCRATCH_LIMIT = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_LAYOUT_NK, MOE_LAYOUT_KN = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_DSWIGLU, MOE_EPI_SWIGLU_MX = 0, 1, 2, 3
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_GROUPS = 256, 32, 1024
MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES = 4 << 20

# exported symbols and their C signatures (mirrors include/moe.h)
_c = ctypes
_P, _I32, _I64, _SZ = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_size_t
SIGNATURES = {
    "moe_abi_version": (_I32, []),
    "moe_status_str": (_c.c_char_p, [_I32]),
    "moe_route_workspace_size": (_I32, [_I64, _I32, _c.POINTER(_SZ)]),
    "moe_router_logits": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _P, _P]),
    "moe_route": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (_I32, [_P, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm": (_I32, [_P, _P, _I32, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_workspace_size": (_I32, [_c.POINTER(_SZ)]),
    "moe_grouped_gemm_gather": (_I32, [_P, _P, _I64, _I32, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _SZ,
                                       _P]),
    "moe_unpermute_combine": (_I32, [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]),
    "moe_grouped_gemm_wgrad": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P]),
    "moe_router_route_workspace_size": (_I32, [_I64, _I32, _c.POINTER(_SZ)]),
    "moe_router_route": (_I32, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                _P, _SZ, _P]),
    "moe_router_route_noalloc": (_I32, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                        _P, _P]),
    "moe_permute_mx": (_I32, [_P, _P, _I64, _I64, _I32, _P, _P, _P, _P]),
    "moe_mx_quantize": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "moe_grouped_gemm_mx": (_I32, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "moe_route_backward": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P]),
    "moe_router_backward_workspace_size": (_I32, [_I64, _I64, _I32, _I32, _c.POINTER(_SZ)]),
    "moe_router_logits_backward": (_I32, [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with `python -m dropless_mixture_experts_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _call(name: str, *args) -> None:
    st = getattr(load_library(), name)(*args)
    if st != MOE_OK:
        raise MoEError(name, st)


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None for None)."""
    if t is None:
        return None
    return t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dense(name: str, t, dtype=None, shape=None, optional: bool = False, flat: bool = False) -> None:
    """A tensor handed to the library must be a contiguous device tensor of the expected dtype and
    shape (flat: of as many elements): the C ABI receives a bare pointer and trusts both."""
    if t is None:
        _need(optional, f"{name} is required")
        return
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        if flat:
            n = 1
            for v in shape:
                n *= v
            _need(t.numel() == n, f"{name} must hold {n} elements, got {t.numel()}")
        else:
            _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _i32():
    import torch
    return torch.int32


def _f32():
    import torch
    return torch.float32


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def moe_abi_version() -> int:
    return int(load_library().moe_abi_version())


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


moe_status_str = status_str


def moe_route_workspace_size(T: int, E: int) -> int:
    n = ctypes.c_size_t(0)
    _call("moe_route_workspace_size", T, E, ctypes.byref(n))
    return int(n.value)


def moe_router_logits(x, w_router, logits, stream=None) -> None:
    """logits[T, E] (fp32) = x[T, d] . w_router[E, d]^T."""
    T, d = x.shape
    E = w_router.shape[0]
    _dense("x", x)
    _dense("w_router", w_router, x.dtype, (E, d))
    _dense("logits", logits, _f32(), (T, E))
    _call("moe_router_logits", _ptr(x), _ptr(w_router), T, d, E, dtype_code(x), _ptr(logits), _stream(stream))


def moe_route(logits, bias, K: int, score: int, renorm: bool, topk_idx, topk_gate, counts, offsets,
              slot_pos, row_src, ws, stream=None) -> None:
    """Top-K routing + histogram + offsets + stable slot positions (all on the device)."""
    T, E = logits.shape
    _dense("logits", logits, _f32())
    _dense("bias", bias, _f32(), (E,), optional=True, flat=True)
    for n, t, dt, sh in (("topk_idx", topk_idx, _i32(), (T, K)), ("topk_gate", topk_gate, _f32(), (T, K)),
                         ("counts", counts, _i32(), (E,)), ("offsets", offsets, _i32(), (E + 1,)),
                         ("slot_pos", slot_pos, _i32(), (T * K,)), ("row_src", row_src, _i32(), (T * K,))):
        _dense(n, t, dt, sh, flat=True)
    _dense("ws", ws, optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _call("moe_route", _ptr(logits), _ptr(bias), T, E, K, score, int(bool(renorm)), _ptr(topk_idx),
          _ptr(topk_gate), _ptr(counts), _ptr(offsets), _ptr(slot_pos), _ptr(row_src), _ptr(ws), ws_bytes,
          _stream(stream))


def moe_permute(x, K: int, slot_pos, x_perm, row_scale=None, y_perm_dot=None, dgate_out=None,
                stream=None) -> None:
    """x_perm[slot_pos[s]] = (row_scale[s] *) x[s // K]; optional dgate_out[s] = <x[s // K], y_perm_dot[slot_pos[s]]>."""
    T, d = x.shape
    _dense("x", x)
    _dense("slot_pos", slot_pos, _i32(), (T * K,), flat=True)
    _dense("x_perm", x_perm, x.dtype, (T * K, d))
    _dense("row_scale", row_scale, _f32(), optional=True)
    _need(row_scale is None or row_scale.numel() == T * K, "row_scale must hold T*K values")
    _dense("y_perm_dot", y_perm_dot, x.dtype, (T * K, d), optional=True)
    _dense("dgate_out", dgate_out, _f32(), optional=True)
    _need(dgate_out is None or dgate_out.numel() == T * K, "dgate_out must hold T*K values")
    _call("moe_permute", _ptr(x), T, d, K, dtype_code(x), _ptr(slot_pos), _ptr(row_scale), _ptr(y_perm_dot),
          _ptr(dgate_out), _ptr(x_perm), _stream(stream))


def moe_grouped_gemm_workspace_size() -> int:
    n = ctypes.c_size_t(0)
    _call("moe_grouped_gemm_workspace_size", ctypes.byref(n))
    return int(n.value)


def moe_grouped_gemm(A, B, b_layout: int, group_offsets, C, epilogue: int = MOE_EPI_NONE, epi_in=None,
                     epi_save=None, workspace=None, stream=None) -> None:
    """One launch over all groups: C_g = epilogue(A_g . B_g^T (NK) or A_g . B_g (KN)).

    ``workspace``: None or a zero-initialised device buffer of moe_grouped_gemm_workspace_size() bytes."""
    M, Kd = A.shape
    G = B.shape[0]
    N = B.shape[1] if b_layout == MOE_LAYOUT_NK else B.shape[2]
    _dense("A", A)
    _dense("B", B, A.dtype, (G, N, Kd) if b_layout == MOE_LAYOUT_NK else (G, Kd, N))
    _dense("group_offsets", group_offsets, _i32(), (G + 1,), flat=True)
    c_cols = {MOE_EPI_NONE: N, MOE_EPI_SWIGLU: N // 2, MOE_EPI_DSWIGLU: 2 * N}.get(epilogue, N)
    _dense("C", C, A.dtype, (M, c_cols))
    _dense("epi_in", epi_in, A.dtype, (M, 2 * N), optional=epilogue != MOE_EPI_DSWIGLU)
    _dense("epi_save", epi_save, A.dtype, (M, N), optional=True)
    _dense("workspace", workspace, optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("moe_grouped_gemm", _ptr(A), _ptr(B), b_layout, _ptr(group_offsets), M, N, Kd, G, dtype_code(A),
          epilogue, _ptr(epi_in), _ptr(epi_save), _ptr(C), _ptr(workspace), ws_bytes, _stream(stream))


def moe_grouped_gemm_gather(x, row_src, K: int, B, group_offsets, C, epilogue: int = MOE_EPI_NONE,
                            epi_save=None, workspace=None, stream=None) -> None:
    """moe_grouped_gemm (layout NK) on A = x[row_src // K] without materialising A: row r of
    the product reads token row row_src[r] // K of x. Bit-identical to moe_permute followed
    by moe_grouped_gemm; raises MoEError (MOE_UNSUPPORTED) for shapes the gathered form does
    not take."""
    T, Kd = x.shape
    G, N = B.shape[0], B.shape[1]
    _dense("x", x)
    _dense("B", B, x.dtype, (G, N, Kd))
    _dense("row_src", row_src, _i32(), (T * K,), flat=True)
    _dense("group_offsets", group_offsets, _i32(), (G + 1,), flat=True)
    _dense("C", C, x.dtype, (T * K, N // 2 if epilogue == MOE_EPI_SWIGLU else N))
    _dense("epi_save", epi_save, x.dtype, (T * K, N), optional=True)
    _dense("workspace", workspace, optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("moe_grouped_gemm_gather", _ptr(x), _ptr(row_src), T, K, _ptr(B), _ptr(group_offsets), N, Kd, G,
          dtype_code(x), epilogue, _ptr(epi_save), _ptr(C), _ptr(workspace), ws_bytes, _stream(stream))


def moe_unpermute_combine(y_perm, slot_pos, gates, T: int, K: int, y, stream=None) -> None:
    """y[t] = sum_k gates[t, k] * y_perm[slot_pos[t*K + k]] (gates None: unit weights)."""
    d = y_perm.shape[1]
    _dense("y_perm", y_perm, shape=(T * K, d))
    _dense("slot_pos", slot_pos, _i32(), (T * K,), flat=True)
    _dense("gates", gates, _f32(), optional=True)
    _need(gates is None or gates.numel() == T * K, "gates must hold T*K values")
    _dense("y", y, y_perm.dtype, (T, d))
    _call("moe_unpermute_combine", _ptr(y_perm), _ptr(slot_pos), _ptr(gates), T, d, K, dtype_code(y_perm),
          _ptr(y), _stream(stream))


def moe_grouped_gemm_wgrad(X, dY, group_offsets, dW, accumulate: bool = False, stream=None) -> None:
    """dW[g] (fp32) = dY_g^T . X_g over the rows of group g; zeros for empty groups."""
    M, Kd = X.shape
    N = dY.shape[1]
    G = dW.shape[0]
    _dense("X", X)
    _dense("dY", dY, X.dtype, (M, N))
    _dense("group_offsets", group_offsets, _i32(), (G + 1,), flat=True)
    _dense("dW", dW, _f32(), (G, N, Kd))
    _call("moe_grouped_gemm_wgrad", _ptr(X), _ptr(dY), _ptr(group_offsets), M, N, Kd, G, dtype_code(X),
          int(bool(accumulate)), _ptr(dW), _stream(stream))




def moe_route_backward(logits, bias, topk_idx, d_gates, score: int, renorm: bool, d_logits, stream=None) -> None:
    """d_logits[T, E] (fp32) = d_gates back through the gates of moe_route, top-K choice held fixed."""
    T, E = logits.shape
    K = topk_idx.shape[1]
    _dense("logits", logits, _f32())
    _dense("bias", bias, _f32(), (E,), optional=True, flat=True)
    _dense("topk_idx", topk_idx, _i32(), (T, K), flat=True)
    _dense("d_gates", d_gates, _f32(), (T, K), flat=True)
    _dense("d_logits", d_logits, _f32(), (T, E))
    _call("moe_route_backward", _ptr(logits), _ptr(bias), _ptr(topk_idx), _ptr(d_gates), T, E, K, score,
          int(bool(renorm)), _ptr(d_logits), _stream(stream))


def moe_router_backward_workspace_size(T: int, d: int, E: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _call("moe_router_backward_workspace_size", T, d, E, dtype, ctypes.byref(n))
    return int(n.value)


def moe_router_logits_backward(d_logits, x, w_router, d_w_router, dx, ws, accumulate: bool = False,
                               stream=None) -> None:
    """d_w_router[E, d] (fp32) = d_logits^T x and/or dx[T, d] (+)= d_logits w_router."""
    T, d = x.shape
    E = w_router.shape[0]
    _dense("x", x)
    _dense("w_router", w_router, x.dtype, (E, d))
    _dense("d_logits", d_logits, _f32(), (T, E))
    _dense("d_w_router", d_w_router, _f32(), (E, d), optional=True)
    _dense("dx", dx, x.dtype, (T, d), optional=True)
    _dense("ws", ws, optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _call("moe_router_logits_backward", _ptr(d_logits), _ptr(x), _ptr(w_router), T, d, E, dtype_code(x),
          _ptr(d_w_router), _ptr(dx), int(bool(accumulate)), _ptr(ws), ws_bytes, _stream(stream))


def moe_router_route_workspace_size(T: int, E: int) -> int:
    n = ctypes.c_size_t(0)
    _call("moe_router_route_workspace_size", T, E, ctypes.byref(n))
    return int(n.value)


def moe_router_route(x, w_router, bias, K: int, score: int, renorm: bool, logits, topk_idx, topk_gate, counts,
                     offsets, slot_pos, row_src, ws, stream=None) -> None:
    """Fused router product + routing (bf16): the results of moe_router_logits then moe_route."""
    T, d = x.shape
    E = w_router.shape[0]
    _dense("x", x)
    _dense("w_router", w_router, x.dtype, (E, d))
    _dense("bias", bias, _f32(), (E,), optional=True, flat=True)
    _dense("logits", logits, _f32(), (T, E), optional=True)
    for n, t, dt, sh in (("topk_idx", topk_idx, _i32(), (T, K)), ("topk_gate", topk_gate, _f32(), (T, K)),
                         ("counts", counts, _i32(), (E,)), ("offsets", offsets, _i32(), (E + 1,)),
                         ("slot_pos", slot_pos, _i32(), (T * K,)), ("row_src", row_src, _i32(), (T * K,))):
        _dense(n, t, dt, sh, flat=True)
    _dense("ws", ws, optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _call("moe_router_route", _ptr(x), _ptr(w_router), _ptr(bias), T, d, E, K, dtype_code(x), score,
          int(bool(renorm)), _ptr(logits), _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _ptr(offsets),
          _ptr(slot_pos), _ptr(row_src), _ptr(ws), ws_bytes, _stream(stream))


def moe_router_route_noalloc(x, w_router, bias, K: int, score: int, renorm: bool, logits, topk_idx, topk_gate,
                             counts, offsets, slot_pos, row_src, stream=None) -> None:
    """moe_router_route with its workspace in the library's static device array: no allocation.
    Calls that overlap in time on one device race on that array."""
    T, d = x.shape
    E = w_router.shape[0]
    _dense("x", x)
    _dense("w_router", w_router, x.dtype, (E, d))
    _dense("bias", bias, _f32(), (E,), optional=True, flat=True)
    _dense("logits", logits, _f32(), (T, E), optional=True)
    for n, t, dt, sh in (("topk_idx", topk_idx, _i32(), (T, K)), ("topk_gate", topk_gate, _f32(), (T, K)),
                         ("counts", counts, _i32(), (E,)), ("offsets", offsets, _i32(), (E + 1,)),
                         ("slot_pos", slot_pos, _i32(), (T * K,)), ("row_src", row_src, _i32(), (T * K,))):
        _dense(n, t, dt, sh, flat=True)
    _call("moe_router_route_noalloc", _ptr(x), _ptr(w_router), _ptr(bias), T, d, E, K, dtype_code(x), score,
          int(bool(renorm)), _ptr(logits), _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _ptr(offsets),
          _ptr(slot_pos), _ptr(row_src), _stream(stream))


def moe_mx_quantize(x, codes, scales, stream=None) -> None:
    """MXFP8 of the rows of x [R, K] (bf16): codes [R, K] uint8, scales [R, K / 32] uint8."""
    R, K = x.shape
    import torch
    _dense("x", x)
    _dense("codes", codes, torch.uint8, (R, K))
    _dense("scales", scales, torch.uint8, (R, K // 32))
    _call("moe_mx_quantize", _ptr(x), R, K, dtype_code(x), _ptr(codes), _ptr(scales), _stream(stream))


def moe_grouped_gemm_mx(A, A_scales, B, B_scales, group_offsets, C, epilogue: int = MOE_EPI_NONE,
                        C_scales=None, workspace=None, stream=None) -> None:
    """Grouped GEMM on MXFP8 operands: A [M, Kd] codes, B [G, N, Kd] codes; bf16 C, or with
    MOE_EPI_SWIGLU_MX the MXFP8 codes C [M, N/2] and scales C_scales [M, N/64] of H.
    ``workspace``: None or a zero-initialised device buffer of moe_grouped_gemm_workspace_size() bytes."""
    M, Kd = A.shape
    G, N = B.shape[0], B.shape[1]
    import torch
    u8 = torch.uint8
    _dense("A", A, u8)
    _dense("A_scales", A_scales, u8, (M, Kd // 32))
    _dense("B", B, u8, (G, N, Kd))
    _dense("B_scales", B_scales, u8, (G, N, Kd // 32))
    _dense("group_offsets", group_offsets, _i32(), (G + 1,), flat=True)
    if epilogue == MOE_EPI_SWIGLU_MX:
        _dense("C", C, u8, (M, N // 2))
        _dense("C_scales", C_scales, u8, (M, N // 64))
    else:
        _dense("C", C, torch.bfloat16, (M, N // 2 if epilogue == MOE_EPI_SWIGLU else N))
        C_scales = None
    _dense("workspace", workspace, optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("moe_grouped_gemm_mx", _ptr(A), _ptr(A_scales), _ptr(B), _ptr(B_scales), _ptr(group_offsets), M, N, Kd,
          G, epilogue, _ptr(C), _ptr(C_scales), _ptr(workspace), ws_bytes, _stream(stream))


def moe_permute_mx(codes, scales, K: int, slot_pos, codes_perm, scales_perm, stream=None) -> None:
    """Row permute of MXFP8 codes [T, d] and scales [T, d / 32] into expert-contiguous order."""
    T, d = codes.shape
    import torch
    u8 = torch.uint8
    _dense("codes", codes, u8)
    _dense("scales", scales, u8, (T, d // 32))
    _dense("slot_pos", slot_pos, _i32(), (T * K,), flat=True)
    _dense("codes_perm", codes_perm, u8, (T * K, d))
    _dense("scales_perm", scales_perm, u8, (T * K, d // 32))
    _call("moe_permute_mx", _ptr(codes), _ptr(scales), T, d, K, _ptr(slot_pos), _ptr(codes_perm), _ptr(scales_perm),
          _stream(stream))


from .layer import (MoEBuffers, backward_steps, forward_steps, gather_supported, layer_backward,  # noqa: E402,F401
                    layer_forward)
