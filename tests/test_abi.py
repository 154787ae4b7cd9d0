"""CPU checks of the C ABI: the library loads, exports every entry point that
include/moe.h declares, and rejects bad arguments on the host before any
launch.  No kernel runs here."""
import ctypes
import os
import re
import subprocess

import pytest

import dropless_mixture_experts_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["moe_route", "moe_permute", "moe_grouped_gemm", "moe_unpermute_combine",
              "moe_grouped_gemm_wgrad", "moe_router_logits", "moe_route_workspace_size",
              "moe_route_backward", "moe_router_logits_backward", "moe_router_backward_workspace_size",
              "moe_router_route", "moe_router_route_workspace_size", "moe_mx_quantize", "moe_grouped_gemm_mx",
              "moe_permute_mx", "moe_router_route_noalloc", "moe_grouped_gemm_gather",
              "moe_status_str", "moe_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(moe_\w+)$", out, re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(moe.SIGNATURES) == set(_declared())


def test_version_and_status_strings(lib):
    assert moe.moe_abi_version() == 10
    assert moe.status_str(0) == "ok"
    assert "invalid" in moe.status_str(1)
    assert "static scratch" in moe.status_str(moe.MOE_SCRATCH_LIMIT)
    assert moe.status_str(99) == "unknown status"


def test_route_workspace_size():
    assert moe.moe_route_workspace_size(0, 8) == 0
    assert moe.moe_route_workspace_size(8192, 8) == 64 * 8 * 4
    assert moe.moe_route_workspace_size(129, 3) == 256
    with pytest.raises(moe.MoEError):
        moe.moe_route_workspace_size(10, 0)
    with pytest.raises(moe.MoEError):
        moe.moe_route_workspace_size(10, 257)


P = 1 << 20  # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def test_route_rejects_bad_arguments(lib):
    ok_ws = 1 << 20
    args = lambda **kw: dict(dict(logits=P, bias=None, T=100, E=8, K=2, score=0, renorm=1, idx=P, gate=P,  # noqa
                                  counts=P, offsets=P, pos=P, src=P, ws=P, wsb=ok_ws), **kw)

    def call(a):
        return lib.moe_route(a["logits"], a["bias"], a["T"], a["E"], a["K"], a["score"], a["renorm"],
                             a["idx"], a["gate"], a["counts"], a["offsets"], a["pos"], a["src"], a["ws"],
                             a["wsb"], None)
    assert call(args(K=9)) == 1           # K > E
    assert call(args(K=0)) == 1
    assert call(args(E=257, K=2)) == 1    # too many experts
    assert call(args(E=64, K=33)) == 1    # K above the top-K limit
    assert call(args(T=-1)) == 1
    assert call(args(score=2)) == 2       # unknown score function
    assert call(args(logits=None)) == 1
    assert call(args(counts=None)) == 1
    assert call(args(wsb=16)) == 1        # workspace too small
    assert call(args(ws=None)) == 1
    assert call(args(T=1 << 28, K=8)) == 1  # T*K >= 2^31


def test_gemm_rejects_bad_arguments(lib):
    def call(A=P, B=P, lay=0, offs=P, M=512, N=256, Kd=128, G=4, dt=1, epi=0, ein=None, esave=None, C=P,
             ws=None, wsb=0):
        return lib.moe_grouped_gemm(A, B, lay, offs, M, N, Kd, G, dt, epi, ein, esave, C, ws, wsb, None)
    assert call(N=12) == 1
    assert call(Kd=4) == 1
    assert call(G=0) == 1
    assert call(G=moe.MOE_MAX_GROUPS + 1) == 1
    assert call(dt=7) == 2
    assert call(lay=2) == 2
    assert call(epi=3) == 2
    assert call(epi=1, lay=1) == 2        # SwiGLU epilogue needs the N-by-K weight layout
    assert call(epi=1, N=24) == 2         # gate|up halves must be 8-aligned
    assert call(epi=2, ein=None) == 1     # SwiGLU backward needs the saved pre-activations
    assert call(A=P + 4) == 1             # misaligned
    assert call(C=None) == 1
    assert call(ws=P + 8, wsb=1 << 20) == 1  # misaligned workspace
    assert call(M=-1) == 1
    assert call(M=0) == 0                 # nothing to do: returns before any launch


def test_gemm_gather_rejects_bad_arguments(lib):
    def call(x=P, src=P, T=256, K=2, B=P, offs=P, N=256, Kd=128, G=4, dt=1, epi=0, esave=None, C=P,
             ws=None, wsb=0):
        return lib.moe_grouped_gemm_gather(x, src, T, K, B, offs, N, Kd, G, dt, epi, esave, C, ws, wsb, None)
    assert call(K=0) == 1
    assert call(K=33) == 1                # top-K limit
    assert call(T=-1) == 1
    assert call(T=1 << 28, K=8) == 1      # T*K >= 2^31
    assert call(N=12) == 1
    assert call(G=0) == 1
    assert call(dt=0) == 2                # the gathered form is bf16 only
    assert call(dt=7) == 2
    assert call(epi=2) == 2               # no SwiGLU-backward epilogue
    assert call(epi=1, N=24) == 2
    assert call(Kd=96) == 2               # whole 64-element K stages only
    assert call(T=1 << 20, Kd=4096) == 2  # token rows beyond 32-bit DMA offsets
    assert call(N=1 << 20, Kd=4096) == 2  # weight rows beyond 32-bit DMA offsets
    assert call(src=None) == 1
    assert call(x=P + 4) == 1             # misaligned
    assert call(src=P + 2) == 1
    assert call(esave=P + 8, epi=1) == 1
    assert call(C=None) == 1
    assert call(ws=P + 8, wsb=1 << 20) == 1
    assert call(T=0, x=None, src=None, C=None) == 0  # nothing to do: returns before any launch


def test_wgrad_permute_combine_reject_bad_arguments(lib):
    assert lib.moe_grouped_gemm_wgrad(P, P, P, 64, 12, 16, 2, 1, 0, P, None) == 1
    assert lib.moe_grouped_gemm_wgrad(P, P, None, 64, 16, 16, 2, 1, 0, P, None) == 1
    assert lib.moe_grouped_gemm_wgrad(P, P, P, 64, 16, 16, 2, 5, 0, P, None) == 2
    assert lib.moe_permute(P, 10, 12, 2, 1, P, None, None, None, P, None) == 1     # d % 8
    assert lib.moe_permute(P, 10, 16, 2, 1, P, None, P, None, P, None) == 1        # dot without output
    assert lib.moe_permute(P, 10, 16, 33, 1, P, None, None, None, P, None) == 1    # K limit
    assert lib.moe_permute(P, 0, 16, 2, 1, None, None, None, None, None, None) == 0  # empty: no launch
    assert lib.moe_unpermute_combine(P, P, None, 10, 16, 0, 1, P, None) == 1
    assert lib.moe_unpermute_combine(P, None, None, 10, 16, 2, 1, P, None) == 1
    assert lib.moe_unpermute_combine(None, None, None, 0, 16, 2, 1, None, None) == 0
    assert lib.moe_router_logits(P, P, 10, 16, 0, 1, P, None) == 1
    assert lib.moe_router_logits(P, P, 10, 20, 8, 1, P, None) == 1
    assert lib.moe_router_logits(P, P, 10, 16, 8, 3, P, None) == 2
    assert lib.moe_router_logits(None, None, 0, 16, 8, 1, None, None) == 0


def test_router_backward_rejects_bad_arguments(lib):
    # moe_route_backward(logits, bias, idx, d_gates, T, E, K, score, renorm, d_logits, stream)
    assert lib.moe_route_backward(P, None, P, P, 10, 8, 9, 0, 1, P, None) == 1      # K > E
    assert lib.moe_route_backward(P, None, P, P, 10, 257, 2, 0, 1, P, None) == 1    # E limit
    assert lib.moe_route_backward(P, None, P, P, 10, 8, 2, 2, 1, P, None) == 2      # unknown score
    assert lib.moe_route_backward(P, None, None, P, 10, 8, 2, 0, 1, P, None) == 1   # no top-K indices
    assert lib.moe_route_backward(P + 2, None, P, P, 10, 8, 2, 0, 1, P, None) == 1  # misaligned
    assert lib.moe_route_backward(None, None, None, None, 0, 8, 2, 0, 1, None, None) == 0  # empty
    n = ctypes.c_size_t(0)
    assert lib.moe_router_backward_workspace_size(100, 20, 8, 1, ctypes.byref(n)) == 1   # d % 8
    assert lib.moe_router_backward_workspace_size(100, 64, 8, 4, ctypes.byref(n)) == 2
    assert lib.moe_router_backward_workspace_size(100, 64, 8, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.moe_router_backward_workspace_size(0, 64, 8, 1, ctypes.byref(n)) == 0   # no tokens
    assert lib.moe_router_backward_workspace_size(1, 8, 1, 1, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.moe_router_backward_workspace_size(100, 64, 8, 1, ctypes.byref(n)) == 0 and n.value > 0
    need = n.value
    # moe_router_logits_backward(dl, x, w, T, d, E, dtype, dw, dx, acc, ws, ws_bytes, stream)
    assert lib.moe_router_logits_backward(P, P, P, 100, 64, 8, 1, P, P, 0, P, need - 1, None) == 1  # small ws
    assert lib.moe_router_logits_backward(P, P, P, 100, 64, 8, 1, P, P, 0, P + 8, need, None) == 1  # misaligned
    assert lib.moe_router_logits_backward(P, None, P, 100, 64, 8, 1, P, None, 0, P, need, None) == 1  # dWr needs x
    assert lib.moe_router_logits_backward(P, P, None, 100, 64, 8, 1, None, P, 0, P, need, None) == 1  # dx needs Wr
    assert lib.moe_router_logits_backward(P, P, P, 100, 64, 8, 3, P, P, 0, P, need, None) == 2
    assert lib.moe_router_logits_backward(P, P, P, 100, 64, 8, 1, None, None, 0, None, 0, None) == 0  # no output


def test_router_route_rejects_bad_arguments(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_router_route_workspace_size(1000, 8, ctypes.byref(n)) == 0 and n.value >= 32 * 8 * 4
    assert lib.moe_router_route_workspace_size(-1, 8, ctypes.byref(n)) == 1
    ws = n.value

    def rr(T=100, d=64, E=8, K=2, dt=1, score=0, x=P, bias=None, wsb=None):
        return lib.moe_router_route(x, P, bias, T, d, E, K, dt, score, 1, None, P, P, P, P, P, P, P,
                                    ws if wsb is None else wsb, None)
    assert rr(dt=0) == 2                  # fp32 takes the unfused path
    assert rr(score=3) == 2
    assert rr(K=9) == 1                   # K > E
    assert rr(d=12) == 1                  # d % 8
    assert rr(x=P + 8) == 1               # misaligned
    assert rr(bias=P + 2) == 1
    assert rr(wsb=0) == 1                 # workspace too small
    assert rr(x=None) == 1


def test_router_route_noalloc_rejects_bad_arguments_and_oversized_inputs(lib):
    def rr(T=100, d=64, E=8, K=2, dt=1, score=0, x=P, bias=None):
        return lib.moe_router_route_noalloc(x, P, bias, T, d, E, K, dt, score, 1, None, P, P, P, P, P, P, None)
    assert rr(dt=0) == 2
    assert rr(score=3) == 2
    assert rr(K=9) == 1
    assert rr(d=12) == 1
    assert rr(x=P + 8) == 1
    assert rr(x=None) == 1
    limit = moe.MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES
    assert limit == 4 << 20
    # the largest inputs whose workspace fits, and the first that do not (ceil(T / 32) E 4 bytes)
    assert moe.moe_router_route_workspace_size(131072, 256) <= limit
    assert moe.moe_router_route_workspace_size(131104, 256) > limit
    assert rr(T=131104, E=256) == moe.MOE_SCRATCH_LIMIT
    assert rr(T=4194336, E=8) == moe.MOE_SCRATCH_LIMIT


def test_mx_rejects_bad_arguments(lib):
    assert lib.moe_mx_quantize(P, 10, 48, 1, P, P, None) == 1          # K % 32
    assert lib.moe_mx_quantize(P, 10, 64, 0, P, P, None) == 2          # bf16 input only
    assert lib.moe_mx_quantize(P + 8, 10, 64, 1, P, P, None) == 1      # misaligned
    assert lib.moe_mx_quantize(None, 0, 64, 1, None, None, None) == 0  # empty: no launch

    def gm(M=64, N=64, Kd=256, G=2, epi=0, A=P, SA=P):
        return lib.moe_grouped_gemm_mx(A, SA, P, P, P, M, N, Kd, G, epi, P, P, None, 0, None)
    assert gm(Kd=192) == 1                 # Kd % 128
    assert gm(epi=2) == 2                  # no SwiGLU-backward epilogue
    assert gm(epi=1, N=24) == 1            # gate|up halves of 8
    assert gm(G=0) == 1
    assert gm(A=P + 4) == 1
    assert gm(SA=P + 2) == 1
    assert gm(N=1 << 20, Kd=1 << 13) == 1  # per-lane offsets past 32 bits
    assert lib.moe_grouped_gemm_mx(P, P, P, P, P, 64, 64, 256, 2, 0, P, None, P + 8, 1 << 30, None) == 1  # workspace alignment
    assert gm(epi=3, N=96) == 1            # MXFP8 H: whole 32-value blocks of F = N / 2
    assert lib.moe_grouped_gemm_mx(P, P, P, P, P, 64, 128, 256, 2, 3, P, None, None, 0, None) == 1  # no C_scales
    assert gm(epi=4) == 2
    assert gm(M=0) == 0
    assert lib.moe_permute_mx(P, P, 10, 256, 2, P, P, P, None) == 1        # d % 512
    assert lib.moe_permute_mx(P, P + 4, 10, 512, 2, P, P, P, None) == 1    # misaligned scales
    assert lib.moe_permute_mx(None, None, 0, 512, 2, None, None, None, None) == 0
