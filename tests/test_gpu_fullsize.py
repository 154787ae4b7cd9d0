"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot run these layers whole, so it checks what it can compute one
by one: the complete routing (indices, counts, offsets, permutation) bit for
bit, the router logits of every token, and the outputs of a seeded sample of
tokens (each token's result depends only on that token and the weights), plus
sampled entries of the weight gradients with the kernels fed seeded inputs of
the backward shapes.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as orc
from tests.gpu_util import GATE_ATOL, TOL_BF16, dev, f64, host, rel_err

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("dropless_mixture_experts_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample(T, n, seed):
    return np.sort(np.random.default_rng(seed).choice(T, size=n, replace=False))


def _forward_full(cfg, logits=None, backward=False):
    inp = mi.make(cfg)
    dv = {k: dev(v) for k, v in inp.items()}
    bufs = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, torch.bfloat16, backward=backward)
    print(f"[fullsize] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} K={cfg.K} F={cfg.F}", flush=True)
    moe.layer_forward(dv["x"], dv["w_router"], dv["bias"], dv["w13"], dv["w2"], cfg.K, cfg.score, cfg.renorm,
                      bufs, logits=dev(logits) if logits is not None else None)
    torch.cuda.synchronize()
    return inp, dv, bufs


@pytest.mark.parametrize("name", ["mixtral", "fine_grained", "dsv3_share"])
def test_full_forward(name):
    cfg = mi.CONFIGS[name]
    inp0 = mi.make(cfg, weights=False)
    logits = orc.router_logits(inp0["x"], inp0["w_router"])
    inp, dv, bufs = _forward_full(cfg, logits=logits)

    # the router product of every token
    gl = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(dv["x"], dv["w_router"], gl)
    torch.cuda.synchronize()
    scale = np.abs(orc.to_f64(inp["x"])) @ np.abs(orc.to_f64(inp["w_router"])).T
    assert np.all(np.abs(host(gl).astype(np.float64) - logits) <= 1e-5 * scale)

    # the whole routing, bit for bit
    r = orc.route(logits, inp["bias"], cfg.K, cfg.score, cfg.renorm)
    np.testing.assert_array_equal(host(bufs.topk_idx), r.idx)
    np.testing.assert_array_equal(host(bufs.counts), r.counts)
    np.testing.assert_array_equal(host(bufs.offsets), r.offsets)
    np.testing.assert_array_equal(host(bufs.slot_pos), r.slot_pos)
    np.testing.assert_array_equal(host(bufs.row_src), r.row_src)
    np.testing.assert_allclose(host(bufs.gates), r.gates, atol=GATE_ATOL, rtol=0)
    if name == "dsv3_share":
        assert (r.counts == 0).sum() == 4

    # sampled tokens through the oracle (routing of a token depends only on its own logits)
    S = _sample(cfg.T, 24, 7)
    ref = orc.forward(inp["x"][S], None, inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm,
                      logits=logits[S])
    assert rel_err(f64(bufs.y)[S], ref["y"]) < TOL_BF16
    # the grouped GEMM rows of the sampled slots (gate/up + SwiGLU output and down output)
    rows = np.array([r.slot_pos[t * cfg.K + k] for t in S for k in range(cfg.K)])
    sub_rows = np.array([ref["routing"].slot_pos[i * cfg.K + k] for i in range(len(S)) for k in range(cfg.K)])
    assert np.array_equal(host(bufs.x_perm)[rows], ref["x_perm"][sub_rows])
    assert rel_err(f64(bufs.h)[rows], ref["h"][sub_rows]) < TOL_BF16
    assert rel_err(f64(bufs.y_perm)[rows], ref["y_perm"][sub_rows]) < TOL_BF16


def test_full_backward_adversarial_skew():
    """Backward of the Mixtral-shaped layer with one expert taking half of the slots
    and two experts none."""
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    inp0 = mi.make(cfg, weights=False)
    hot, dead = mi.skew_choice(cfg)
    logits = mi.skew_logits(orc.router_logits(inp0["x"], inp0["w_router"]), hot, dead)
    inp, dv, bufs = _forward_full(cfg, logits=logits, backward=True)
    dy = mi.upstream_grad(cfg)
    moe.layer_backward(dev(dy), dv["w13"], dv["w2"], cfg.K, bufs)
    torch.cuda.synchronize()

    counts = host(bufs.counts)
    assert counts[hot] == cfg.T and all(counts[e] == 0 for e in dead)
    assert counts.sum() == cfg.T * cfg.K
    dw13, dw2 = bufs.dw13, bufs.dw2
    for e in dead:
        assert not torch.any(dw13[e]).item() and not torch.any(dw2[e]).item()

    S = _sample(cfg.T, 16, 11)
    fwd = orc.forward(inp["x"][S], None, None, inp["w13"], inp["w2"], cfg.K, logits=logits[S])
    bwd = orc.backward(dy[S], fwd, inp["w13"], inp["w2"], cfg.K)
    assert rel_err(f64(bufs.y)[S], fwd["y"]) < TOL_BF16
    assert rel_err(f64(bufs.dx)[S], bwd["dx"]) < TOL_BF16
    assert rel_err(f64(bufs.d_gates)[S], bwd["d_gates"]) < TOL_BF16


def _c5_offsets():
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    hot, dead = mi.skew_choice(cfg)
    M = cfg.T * cfg.K
    counts = np.zeros(cfg.E, np.int64)
    counts[hot] = cfg.T
    rest = [e for e in range(cfg.E) if e != hot and e not in dead]
    base = (M - cfg.T) // len(rest)
    for i, e in enumerate(rest):
        counts[e] = base + (1 if i < (M - cfg.T) - base * len(rest) else 0)
    return np.concatenate([[0], np.cumsum(counts)]), counts


@pytest.mark.parametrize("which", ["down", "gate_up"])
def test_full_wgrad_backward_shapes(which):
    """dW_e = dY_e^T X_e at the backward shapes (hot group of 8192 rows, five of ~1638,
    two empty), seeded inputs; sampled entries against the oracle, empty groups exactly 0."""
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    off, counts = _c5_offsets()
    M = int(off[-1])
    if which == "down":      # dW2 [E, d, F] = dY_perm^T H
        Kd, N = cfg.F, cfg.d
    else:                    # dW13 [E, 2F, d] = dA^T X_perm
        Kd, N = cfg.d, 2 * cfg.F
    X = mi.normal(91, 1, (M, Kd), 1.0, True)
    dY = mi.normal(91, 2, (M, N), 1.0, True)
    dW = torch.empty((cfg.E, N, Kd), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm_wgrad(dev(X), dev(dY), dev(off), dW)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ncols = rng.choice(N, 24, replace=False)
    kcols = rng.choice(Kd, 24, replace=False)
    ref = orc.grouped_wgrad(X[:, kcols], dY[:, ncols], off)      # [E, 24, 24]
    got = dW[:, torch.as_tensor(ncols, device="cuda")][:, :, torch.as_tensor(kcols, device="cuda")]
    got = host(got).astype(np.float64)
    for e in range(cfg.E):
        if counts[e] == 0:
            assert not torch.any(dW[e]).item()
        else:
            assert rel_err(got[e], ref[e]) < TOL_BF16 / 4, e


def test_full_dgrad_swiglu_backward_shapes():
    """dA = SwiGLU'(dY_perm . W2, saved pre-activations) in the K-by-N weight layout at
    the backward shapes; sampled rows against the oracle."""
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    off, counts = _c5_offsets()
    M = int(off[-1])
    dYp = mi.normal(92, 1, (M, cfg.d), 1.0, True)
    pre = mi.normal(92, 2, (M, 2 * cfg.F), 1.0, True)
    w2 = mi.normal(cfg.seed, mi.TAG_W2, (cfg.E, cfg.d, cfg.F), 1.0 / 64, True)
    dA = torch.empty((M, 2 * cfg.F), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(dev(dYp), dev(w2), moe.MOE_LAYOUT_KN, dev(off), dA, moe.MOE_EPI_DSWIGLU,
                         epi_in=dev(pre))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(M, 32, replace=False))
    got = f64(dA)[rows]
    grp = np.searchsorted(off, rows, side="right") - 1
    for e in np.unique(grp):
        sel = np.nonzero(grp == e)[0]
        dh = orc.grouped_gemm(dYp[rows[sel]], w2[e:e + 1], np.array([0, len(sel)]), "kn")
        ref = orc.swiglu_backward(dh, pre[rows[sel]])
        assert rel_err(got[sel], ref) < TOL_BF16, e
