"""GPU parity over seeded random shapes of the grouped GEMM paths the layer uses: the N-by-K
ring (plain and SwiGLU, on a permuted copy or on gathered token rows), the K-by-N ring (plain and
SwiGLU backward), and the weight gradient,
against the CPU oracle.  Each case draws a group count, ragged group sizes with empty and
dominant groups, widths and reduction lengths spanning several tiles with ragged tails, rows
outside the groups, and whether a workspace (the split tail) is passed.  Bars as in the other
parity tests: relative Frobenius error within 2e-2 / 4 over the groups' rows, 2e-2 row by row,
rows outside the groups untouched, empty groups' weight gradients exactly zero.
"""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as orc
from tests.gpu_util import TOL_BF16, dev, empty_like_poisoned, f64, rel_err

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("dropless_mixture_experts_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _counts(rng, G, mean):
    """Ragged group sizes: a quarter of the groups empty, one group dominant, the rest spread."""
    c = rng.integers(0, 2 * mean + 1, size=G)
    c[rng.random(G) < 0.25] = 0
    c[rng.integers(G)] += int(rng.integers(mean, 4 * mean + 1))
    return c


def _case(seed, N, Kd, mean, gmax=24):
    rng = np.random.default_rng(seed)
    G = int(rng.integers(1, gmax + 1))
    counts = _counts(rng, G, mean)
    lead, tail = int(rng.integers(0, 9)), int(rng.integers(0, 9))
    off = lead + np.concatenate([[0], np.cumsum(counts)])
    M = int(off[-1]) + tail
    A = mi.f32_to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    W = mi.f32_to_bf16_bits((rng.standard_normal((G, N, Kd)) / math.sqrt(Kd)).astype(np.float32))
    use_ws = bool(rng.integers(2))
    return rng, A, W, off, M, use_ws


def _check_rows(C, off, M, ref):
    c = f64(C)
    lo, hi = int(off[0]), int(off[-1])
    assert np.all(np.isnan(c[:lo])) and np.all(np.isnan(c[hi:M])), "rows outside the groups written"
    got = c[lo:hi]
    assert not np.any(np.isnan(got))
    if hi > lo:
        assert rel_err(got, ref) < TOL_BF16 / 4
        row = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        assert row.max() < TOL_BF16


def _workspace(use):
    if not use:
        return None
    return torch.zeros((moe.moe_grouped_gemm_workspace_size(),), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("seed", range(8))
def test_sweep_nk_plain(seed):
    rng0 = np.random.default_rng(1000 + 500 + seed)
    N = 8 * int(rng0.integers(1, 97))          # 8 .. 768
    Kd = 64 * int(rng0.integers(1, 13))        # 64 .. 768: whole ring stages
    _, A, W, off, M, use_ws = _case(1000 + seed, N, Kd, mean=200)
    C = empty_like_poisoned((M, N), torch.bfloat16)
    ws = _workspace(use_ws)
    moe.moe_grouped_gemm(dev(A), dev(W), 0, dev(off), C, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert torch.count_nonzero(ws[:4096]).item() == 0
    lo = int(off[0])
    _check_rows(C, off, M, orc.grouped_gemm(A[lo:int(off[-1])], W, off - lo, "nk"))


@pytest.mark.parametrize("seed", range(8))
def test_sweep_nk_swiglu(seed):
    rng0 = np.random.default_rng(2000 + 500 + seed)
    F = 8 * int(rng0.integers(1, 65))          # 8 .. 512
    Kd = 64 * int(rng0.integers(1, 13))
    _, A, W, off, M, use_ws = _case(2000 + seed, 2 * F, Kd, mean=200)
    H = empty_like_poisoned((M, F), torch.bfloat16)
    P = empty_like_poisoned((M, 2 * F), torch.bfloat16)
    moe.moe_grouped_gemm(dev(A), dev(W), 0, dev(off), H, moe.MOE_EPI_SWIGLU, epi_save=P,
                         workspace=_workspace(use_ws))
    torch.cuda.synchronize()
    lo = int(off[0])
    pre = orc.grouped_gemm(A[lo:int(off[-1])], W, off - lo, "nk")
    _check_rows(H, off, M, orc.swiglu(pre))
    _check_rows(P, off, M, pre)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_gather(seed):
    """The gate/up GEMM on gathered token rows (plain or SwiGLU, with or without the split-tail
    workspace) over random routings: bit-identical to moe_permute followed by moe_grouped_gemm,
    and within the bars of the oracle on the permuted rows."""
    rng = np.random.default_rng(2500 + seed)
    T, E = int(rng.integers(1, 3000)), int(rng.integers(1, 65))
    K = int(rng.integers(1, min(E, 8) + 1))
    Kd = 64 * int(rng.integers(1, 13))
    swiglu = bool(rng.integers(2))
    N = 16 * int(rng.integers(1, 49)) if swiglu else 8 * int(rng.integers(1, 97))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = orc.route(logits, None, K)
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, Kd)).astype(np.float32))
    W = mi.f32_to_bf16_bits((rng.standard_normal((E, N, Kd)) / math.sqrt(Kd)).astype(np.float32))
    ws = _workspace(bool(rng.integers(2)))
    epi = moe.MOE_EPI_SWIGLU if swiglu else moe.MOE_EPI_NONE
    width = N // 2 if swiglu else N
    M = T * K
    xd, Wd, offs = dev(x), dev(W), dev(r.offsets)
    C = empty_like_poisoned((M, width), torch.bfloat16)
    moe.moe_grouped_gemm_gather(xd, dev(r.row_src), K, Wd, offs, C, epi, workspace=ws)
    xp = empty_like_poisoned((M, Kd), torch.bfloat16)
    moe.moe_permute(xd, K, dev(r.slot_pos), xp)
    C2 = empty_like_poisoned((M, width), torch.bfloat16)
    moe.moe_grouped_gemm(xp, Wd, 0, offs, C2, epi, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    pre = orc.grouped_gemm(orc.permute(x, r.row_src, K), W, r.offsets, "nk")
    _check_rows(C, r.offsets, M, orc.swiglu(pre) if swiglu else pre)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_kn_plain(seed):
    rng0 = np.random.default_rng(3000 + 500 + seed)
    N = 8 * int(rng0.integers(1, 97))
    Kd = 64 * int(rng0.integers(1, 13))
    _, A, W, off, M, use_ws = _case(3000 + seed, N, Kd, mean=200)
    Wkn = np.ascontiguousarray(W.transpose(0, 2, 1))   # [G, Kd, N]
    C = empty_like_poisoned((M, N), torch.bfloat16)
    moe.moe_grouped_gemm(dev(A), dev(Wkn), 1, dev(off), C, workspace=_workspace(use_ws))
    torch.cuda.synchronize()
    lo = int(off[0])
    _check_rows(C, off, M, orc.grouped_gemm(A[lo:int(off[-1])], Wkn, off - lo, "kn"))


@pytest.mark.parametrize("seed", range(8))
def test_sweep_kn_dswiglu(seed):
    rng0 = np.random.default_rng(4000 + 500 + seed)
    F = 8 * int(rng0.integers(1, 65))
    Kd = 64 * int(rng0.integers(1, 13))
    rng, A, W, off, M, use_ws = _case(4000 + seed, F, Kd, mean=200)
    Wkn = np.ascontiguousarray(W.transpose(0, 2, 1))   # [G, Kd, F]
    pre = mi.f32_to_bf16_bits(rng.standard_normal((M, 2 * F)).astype(np.float32))
    C = empty_like_poisoned((M, 2 * F), torch.bfloat16)
    moe.moe_grouped_gemm(dev(A), dev(Wkn), 1, dev(off), C, moe.MOE_EPI_DSWIGLU, epi_in=dev(pre),
                         workspace=_workspace(use_ws))
    torch.cuda.synchronize()
    lo, hi = int(off[0]), int(off[-1])
    dh = orc.grouped_gemm(A[lo:hi], Wkn, off - lo, "kn")
    _check_rows(C, off, M, orc.swiglu_backward(dh, pre[lo:hi]))


@pytest.mark.parametrize("seed", range(8))
def test_sweep_wgrad(seed):
    rng = np.random.default_rng(5000 + seed)
    G = int(rng.integers(1, 17))
    counts = _counts(rng, G, 150)
    off = np.concatenate([[0], np.cumsum(counts)])
    M = int(off[-1])
    N = 8 * int(rng.integers(1, 97))
    Kd = 8 * int(rng.integers(1, 97))
    accumulate = bool(rng.integers(2))
    X = mi.f32_to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    dY = mi.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    init = rng.standard_normal((G, N, Kd)).astype(np.float32)
    dW = dev(init) if accumulate else empty_like_poisoned((G, N, Kd), torch.float32)
    moe.moe_grouped_gemm_wgrad(dev(X), dev(dY), dev(off), dW, accumulate=accumulate)
    torch.cuda.synchronize()
    got = f64(dW)
    ref = orc.grouped_wgrad(X, dY, off) + (init.astype(np.float64) if accumulate else 0.0)
    for g in range(G):
        if counts[g] == 0:
            assert np.array_equal(got[g], ref[g]), "an empty group's gradient must be zero (or untouched)"
        else:
            assert rel_err(got[g], ref[g]) < TOL_BF16 / 4, g


def _route_case(rng, E, K):
    """A bias for half the cases, with up to E - K experts masked by -inf (K finite keys remain)."""
    if not rng.integers(2):
        return None
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32)
    bias[rng.choice(E, int(rng.integers(0, E - K + 1)), replace=False)] = -np.inf
    return bias


@pytest.mark.parametrize("seed", range(12))
def test_sweep_route(seed):
    """Routing of random logits: indices, counts, offsets, slot positions and the permutation
    bit-exact against the oracle, gates within 1e-5."""
    from tests.test_gpu_parity import _check_route
    rng = np.random.default_rng(6000 + seed)
    E = int(rng.integers(1, 257))
    K = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.integers(1, 6000))
    score, renorm = int(rng.integers(2)), bool(rng.integers(2))
    logits = (rng.standard_normal((T, E)) * rng.uniform(0.1, 3.0)).astype(np.float32)
    _check_route(logits, _route_case(rng, E, K), K, score, renorm)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_router_route(seed):
    """The fused router equals the router product followed by routing (every output bit for
    bit), and routes the tokens with a clear top-K margin as the oracle does."""
    from tests.test_gpu_parity import _check_route_clear_tokens, _fused_vs_unfused
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(1, 257))
    K = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.integers(1, 20000))
    d = 8 * int(rng.integers(1, 257))
    score, renorm = int(rng.integers(2)), bool(rng.integers(2))
    bias = _route_case(rng, E, K)
    x, w, idx, gate = _fused_vs_unfused(T, d, E, K, score, renorm, bias=bias, seed=7100 + seed)
    _check_route_clear_tokens(x, w, bias, K, score, renorm, idx, gate)


@pytest.mark.parametrize("seed", range(6))
def test_sweep_mx_quantize(seed):
    """MX block quantisation of random rows with per-row magnitudes from 2^-30 to 2^30: codes
    and scales bit-exact against the oracle."""
    rng = np.random.default_rng(8000 + seed)
    R, K = int(rng.integers(1, 3000)), 32 * int(rng.integers(1, 129))
    v = rng.standard_normal((R, K)) * np.exp2(rng.integers(-30, 31, (R, 1)))
    v[rng.random((R, K)) < 0.01] = 0.0
    x = mi.f32_to_bf16_bits(v.astype(np.float32))
    codes = torch.full((R, K), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((R, K // 32), 0xAA, dtype=torch.uint8, device="cuda")
    moe.moe_mx_quantize(dev(x), codes, scales)
    torch.cuda.synchronize()
    rc, rs = orc.mx_quantize(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("seed", range(8))
def test_sweep_grouped_gemm_mx(seed):
    """The MX grouped GEMM on random group loads, widths and reduction lengths, plain or SwiGLU,
    against the oracle's product of the same codes and scales."""
    from tests.test_gpu_parity import _check_mx_gemm, _mx_operands
    rng = np.random.default_rng(9000 + seed)
    G = int(rng.integers(1, 13))
    counts = _counts(rng, G, 150)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offs[-1])
    epi = int(rng.integers(2))
    N = 16 * int(rng.integers(1, 49))           # 16 .. 768
    Kd = 128 * int(rng.integers(1, 9))          # 128 .. 1024
    ac, asc = _mx_operands(rng, M, Kd)
    bc, bsc = _mx_operands(rng, G * N, Kd)
    C = torch.full((M, N // 2 if epi == 1 else N), float("nan"), dtype=torch.bfloat16, device="cuda")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = _workspace(bool(rng.integers(2)))
    moe.moe_grouped_gemm_mx(u8(ac), u8(asc), u8(bc.reshape(G, N, Kd)), u8(bsc.reshape(G, N, Kd // 32)),
                            dev(offs), C, epilogue=epi, workspace=ws)
    torch.cuda.synchronize()
    _check_mx_gemm(ac, asc, bc, bsc, G, N, Kd, offs, C, epi)
    if ws is not None:
        assert torch.count_nonzero(ws[:4096]).item() == 0
    if epi == 1 and N % 64 == 0:
        # H written as MXFP8 by the epilogue: the bytes of quantising the bf16 H above
        F = N // 2
        hc, hs = torch.empty((M, F), dtype=torch.uint8, device="cuda"), torch.empty((M, F // 32), dtype=torch.uint8, device="cuda")
        moe.moe_mx_quantize(C, hc, hs)
        qc, qs = torch.empty_like(hc), torch.empty_like(hs)
        moe.moe_grouped_gemm_mx(u8(ac), u8(asc), u8(bc.reshape(G, N, Kd)), u8(bsc.reshape(G, N, Kd // 32)),
                                dev(offs), qc, epilogue=moe.MOE_EPI_SWIGLU_MX, C_scales=qs, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(qc, hc) and torch.equal(qs, hs)


@pytest.mark.parametrize("seed", range(6))
def test_sweep_layer_forward_backward(seed):
    """The whole layer, forward and backward with the router backward, on random small
    configurations (routing on the oracle's fp32 logits so that it is exact): outputs and every
    gradient against the oracle; empty experts' weight gradients exactly zero."""
    from tests.test_gpu_parity import _run_layer
    rng = np.random.default_rng(10000 + seed)
    E = int(rng.integers(1, 65))
    K = int(rng.integers(1, min(E, 8) + 1))
    cfg = mi.MoEConfig(f"sweep_{seed}", seed=10100 + seed, T=int(rng.integers(16, 1500)),
                       d=64 * int(rng.integers(1, 9)), E=E, K=K, F=8 * int(rng.integers(8, 65)), bf16=True,
                       score=int(rng.integers(2)), renorm=bool(rng.integers(2)), wr_std=0.05,
                       dy_seed=10200 + seed)
    inp = mi.make(cfg)
    logits = orc.router_logits(inp["x"], inp["w_router"])
    dy = mi.upstream_grad(cfg)
    bufs, dv = _run_layer(cfg, inp, logits=logits, backward=True)
    router = dict(logits=dev(logits), x=dv["x"], w_router=dv["w_router"], bias=None, score=cfg.score,
                  renorm=cfg.renorm)
    moe.layer_backward(dev(dy), dv["w13"], dv["w2"], cfg.K, bufs, router=router)
    torch.cuda.synchronize()
    fwd = orc.forward(inp["x"], None, None, inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm, logits=logits)
    bwd = orc.backward(dy, fwd, inp["w13"], inp["w2"], cfg.K)
    r = fwd["routing"]
    np.testing.assert_array_equal(host_i(bufs.topk_idx), r.idx)
    np.testing.assert_array_equal(host_i(bufs.counts), r.counts)
    d_logits = orc.route_backward(logits, r.idx, bwd["d_gates"], cfg.score, cfg.renorm)
    dwr, dx_router = orc.router_backward(d_logits, inp["x"], inp["w_router"])
    assert rel_err(bufs.y, fwd["y"]) < TOL_BF16
    assert rel_err(bufs.d_gates, bwd["d_gates"]) < TOL_BF16
    assert rel_err(bufs.dx, bwd["dx"] + dx_router) < TOL_BF16
    assert rel_err(bufs.d_logits, d_logits) < TOL_BF16
    assert rel_err(bufs.dw_router, dwr) < TOL_BF16
    dw13, dw2 = f64(bufs.dw13), f64(bufs.dw2)
    for e in range(cfg.E):
        if r.counts[e] == 0:
            assert not np.any(dw13[e]) and not np.any(dw2[e]), e
        else:
            assert rel_err(dw13[e], bwd["dw13"][e]) < TOL_BF16, e
            assert rel_err(dw2[e], bwd["dw2"][e]) < TOL_BF16, e


def host_i(t):
    return t.detach().cpu().numpy()
