"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a hand-derived value, a closed form, a
library routine for a special case, brute force on tiny inputs, or an
invariant of the method, so that a dropped term, a wrong sign or index or a
transposed operand anywhere in it fails at least one test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import moe_inputs as mi
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _tiny(T=48, d=16, E=6, K=2, F=8, seed=11, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    w13 = (rng.standard_normal((E, 2 * F, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, d, F)) / math.sqrt(F)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    return x, wr, w13, w2, b


# ---------------------------------------------------------------- value decoding

def test_to_f64_decodes_bf16_bit_patterns():
    """bf16 is the upper half of an IEEE binary32: sign, 8 exponent bits (bias 127), 7 mantissa bits."""
    table = {0x3F80: 1.0, 0xBF80: -1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x3E80: 0.25,
             0x0000: 0.0, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
             0x0001: 2.0 ** -133, 0x807F: -(1.0 - 2.0 ** -7) * 2.0 ** -126,
             0x7F80: math.inf, 0xFF80: -math.inf}
    codes = np.array(list(table), dtype=np.uint16)
    got = orc.to_f64(codes)
    assert got.dtype == np.float64
    assert got.tolist() == list(table.values())
    neg0 = orc.to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    assert np.isnan(orc.to_f64(np.array([0x7FC0, 0xFFC1], np.uint16))).all()
    # fp32 and fp64 inputs are widened exactly
    f = np.array([0.1, -3.5e-40], np.float32)
    assert orc.to_f64(f).tolist() == [float(v) for v in f]


# ---------------------------------------------------------------- worked examples

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_single_expert_swiglu():
    c = _golden()["single_expert_swiglu"]
    out = orc.forward(np.array(c["x"], np.float32), None, None, np.array(c["w13"], np.float32),
                      np.array(c["w2"], np.float32), c["K"], logits=np.array(c["logits"], np.float32))
    assert out["routing"].idx.tolist() == c["expect_idx"]
    assert out["routing"].gates.tolist() == c["expect_gates"]
    np.testing.assert_allclose(out["h"], c["expect_h"], rtol=1e-14)
    np.testing.assert_allclose(out["y"], c["expect_y"], rtol=1e-14)


def test_worked_example_two_tokens_two_experts():
    c = _golden()["two_tokens_two_experts"]
    out = orc.forward(np.array(c["x"], np.float32), None, None, np.array(c["w13"], np.float32),
                      np.array(c["w2"], np.float32), c["K"], logits=np.array(c["logits"], np.float32))
    r = out["routing"]
    assert r.idx.tolist() == c["expect_idx"]
    # ln 3 is rounded to fp32 in the logits, so the gates are 3/4, 1/4 within ~1e-7
    np.testing.assert_allclose(r.gates, c["expect_gates"], atol=1e-7)
    assert r.counts.tolist() == c["expect_counts"]
    assert r.offsets.tolist() == c["expect_offsets"]
    assert r.row_src.tolist() == c["expect_row_src"]
    assert r.slot_pos.tolist() == c["expect_slot_pos"]
    np.testing.assert_allclose(out["y"], c["expect_y"], rtol=1e-6)


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("K", [1, 2, 3, 6])
@pytest.mark.parametrize("score", [orc.SCORE_SOFTMAX, orc.SCORE_SIGMOID])
def test_topk_matches_brute_force_over_subsets(K, score):
    rng = np.random.default_rng(100 + K)
    T, E = 40, 6
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = orc.route(logits, None, K, score)
    for t in range(T):
        best = max(itertools.combinations(range(E), K),
                   key=lambda S: sum(float(logits[t, e]) for e in S))
        assert set(r.idx[t].tolist()) == set(best)
        ks = logits[t, r.idx[t]]
        assert np.all(ks[:-1] > ks[1:]), "chosen experts must be listed by descending key"
        assert len(set(r.idx[t].tolist())) == K


def test_tie_break_lower_expert_first_and_signed_zero():
    keys = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    assert orc.route(keys, None, 2).idx.tolist() == [[1, 2]]
    assert orc.route(keys, None, 3).idx.tolist() == [[1, 2, 3]]
    z = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert orc.route(z, None, 1).idx.tolist() == [[1]]
    allsame = np.zeros((1, 5), np.float32)
    assert orc.route(allsame, None, 3).idx.tolist() == [[0, 1, 2]]


def test_gates_closed_forms_softmax():
    rng = np.random.default_rng(7)
    T, E, K = 30, 8, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = orc.route(logits, None, K, orc.SCORE_SOFTMAX, renorm=True)
    for t in range(T):
        # renormalised softmax over all E == softmax over the K chosen keys
        ref = softmax(logits[t, r.idx[t]].astype(np.float64))
        np.testing.assert_allclose(r.gates[t], ref, rtol=1e-12)
    np.testing.assert_allclose(r.gates.sum(1), 1.0, rtol=1e-12)
    # without renormalisation the gates are the full softmax at the chosen experts
    r2 = orc.route(logits, None, K, orc.SCORE_SOFTMAX, renorm=False)
    full = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(r2.gates, np.take_along_axis(full, r2.idx.astype(np.int64), 1), rtol=1e-12)
    # K = E: the renormalised gates are the full softmax in key order
    r3 = orc.route(logits, None, E)
    np.testing.assert_allclose(r3.gates, np.take_along_axis(full, r3.idx.astype(np.int64), 1), rtol=1e-12)
    # K = 1: the gate is exactly 1
    assert np.all(orc.route(logits, None, 1).gates == 1.0)


def test_gates_closed_forms_sigmoid():
    rng = np.random.default_rng(8)
    T, E, K = 30, 8, 4
    logits = (2 * rng.standard_normal((T, E))).astype(np.float32)
    r = orc.route(logits, None, K, orc.SCORE_SIGMOID, renorm=True)
    for t in range(T):
        s = expit(logits[t, r.idx[t]].astype(np.float64))
        np.testing.assert_allclose(r.gates[t], s / s.sum(), rtol=1e-12)
    r2 = orc.route(logits, None, K, orc.SCORE_SIGMOID, renorm=False)
    np.testing.assert_allclose(r2.gates, expit(np.take_along_axis(logits, r2.idx.astype(np.int64), 1)
                                               .astype(np.float64)), rtol=1e-12)


def test_bias_changes_routing_as_predicted():
    """The bias is a non-weight input of its own: it shifts the keys before the
    choice and before the scores."""
    rng = np.random.default_rng(9)
    T, E, K = 64, 8, 2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[5] = 100.0
    b[2] = -np.inf
    r = orc.route(logits, b, K)
    assert np.all(r.idx[:, 0] == 5)
    assert not np.any(r.idx == 2)
    keys = logits + b
    for t in range(T):
        np.testing.assert_allclose(r.gates[t], softmax(keys[t, r.idx[t]].astype(np.float64)), rtol=1e-12)
    # the key add is an fp32 add: the routing sees fp32(logit + bias)
    assert r.keys.dtype == np.float32 and np.array_equal(r.keys, logits + b)


def test_counts_offsets_and_stable_permutation():
    rng = np.random.default_rng(10)
    T, E, K = 200, 7, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 4] -= 3.0  # a rarely chosen expert
    logits[:, 6] = -np.inf  # an expert that gets nothing
    r = orc.route(logits, None, K)
    M = T * K
    assert r.counts.sum() == M
    assert np.array_equal(r.counts, np.bincount(r.idx.ravel(), minlength=E))
    assert r.counts[6] == 0
    assert np.array_equal(r.offsets, np.concatenate([[0], np.cumsum(r.counts)]))
    assert np.array_equal(r.row_src, np.argsort(r.idx.ravel(), kind="stable"))
    assert np.array_equal(r.slot_pos[r.row_src], np.arange(M))
    assert np.array_equal(np.sort(r.slot_pos), np.arange(M))
    for e in range(E):
        toks = r.row_src[r.offsets[e]:r.offsets[e + 1]] // K
        assert np.all(np.diff(toks) > 0)


# ---------------------------------------------------------------- permute / combine

def test_permute_is_a_bit_copy():
    rng = np.random.default_rng(12)
    T, d, E, K = 50, 24, 5, 2
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    r = orc.route(rng.standard_normal((T, E)).astype(np.float32), None, K)
    xp = orc.permute(x, r.row_src, K)
    assert xp.dtype == np.uint16
    assert np.array_equal(xp, x[r.row_src // K])


def test_identity_experts_return_x_times_gate_sum():
    rng = np.random.default_rng(13)
    T, d, E, K = 64, 10, 6, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    r = orc.route(rng.standard_normal((T, E)).astype(np.float32), None, K)
    xp = orc.permute(x, r.row_src, K)
    y = orc.combine(xp, r.slot_pos, r.gates, T, K)
    np.testing.assert_allclose(y, x.astype(np.float64) * r.gates.sum(1, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(y, x.astype(np.float64), rtol=1e-14)
    y1 = orc.combine(xp, r.slot_pos, None, T, K)
    np.testing.assert_array_equal(y1, K * x.astype(np.float64))


def test_permute_and_unit_combine_are_adjoint():
    rng = np.random.default_rng(14)
    T, d, E, K = 40, 6, 5, 2
    x = rng.standard_normal((T, d))
    r = orc.route(rng.standard_normal((T, E)).astype(np.float32), None, K)
    v = rng.standard_normal((T * K, d))
    lhs = float((orc.permute(x, r.row_src, K) * v).sum())
    rhs = float((x * orc.combine(v, r.slot_pos, None, T, K)).sum())
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


# ---------------------------------------------------------------- grouped GEMM

def test_grouped_gemm_single_group_is_plain_matmul():
    rng = np.random.default_rng(15)
    a = rng.standard_normal((37, 12))
    b = rng.standard_normal((1, 9, 12))
    np.testing.assert_allclose(orc.grouped_gemm(a, b, np.array([0, 37])), np.matmul(a, b[0].T), rtol=1e-13)


def test_grouped_gemm_equal_counts_is_batched_gemm():
    rng = np.random.default_rng(16)
    G, m, n, k = 4, 5, 7, 6
    a = rng.standard_normal((G * m, k))
    b = rng.standard_normal((G, n, k))
    ref = np.einsum("gmk,gnk->gmn", a.reshape(G, m, k), b).reshape(G * m, n)
    np.testing.assert_allclose(orc.grouped_gemm(a, b, np.arange(G + 1) * m), ref, rtol=1e-13)
    # the K-by-N layout of the same weights gives the same product
    np.testing.assert_allclose(orc.grouped_gemm(a, np.ascontiguousarray(b.transpose(0, 2, 1)),
                                                np.arange(G + 1) * m, "kn"), ref, rtol=1e-13)


def test_grouped_gemm_scaled_identity_detects_wrong_expert():
    rng = np.random.default_rng(17)
    counts = np.array([3, 0, 5, 1, 4])
    off = np.concatenate([[0], np.cumsum(counts)])
    d = 8
    a = rng.standard_normal((off[-1], d))
    c = np.array([2.0, 4.0, 0.5, 8.0, 0.25])
    b = np.stack([ci * np.eye(d) for ci in c])
    out = orc.grouped_gemm(a, b, off)
    for g in range(5):
        np.testing.assert_array_equal(out[off[g]:off[g + 1]], c[g] * a[off[g]:off[g + 1]])


def test_wgrad_sums_to_one_dense_gemm_and_zero_for_empty_groups():
    rng = np.random.default_rng(18)
    counts = np.array([4, 0, 7, 2])
    off = np.concatenate([[0], np.cumsum(counts)])
    x = rng.standard_normal((off[-1], 5))
    dy = rng.standard_normal((off[-1], 3))
    dW = orc.grouped_wgrad(x, dy, off)
    assert dW.shape == (4, 3, 5)
    np.testing.assert_array_equal(dW[1], 0.0)
    np.testing.assert_allclose(dW.sum(0), dy.T @ x, rtol=1e-12)
    np.testing.assert_allclose(dW[2], sum(np.outer(dy[i], x[i]) for i in range(off[2], off[3])), rtol=1e-12)


def test_swiglu_closed_forms():
    v = np.array([[0.0, 2.0, -2.0, 40.0, 1.0, 3.0, 5.0, 7.0]])   # gate | up
    h = orc.swiglu(v)
    t1 = math.tanh(1.0)
    np.testing.assert_allclose(h, [[0.0, 2 * (1 + t1) / 2 * 3.0, -2 * (1 - t1) / 2 * 5.0, 40.0 * 7.0]], rtol=1e-14)


# ---------------------------------------------------------------- whole layer

@pytest.mark.parametrize("score", [orc.SCORE_SOFTMAX, orc.SCORE_SIGMOID])
def test_layer_matches_dense_masked_evaluation(score):
    x, wr, w13, w2, b = _tiny(bias=True)
    out = orc.forward(x, wr, b, w13, w2, K=2, score=score)
    ref = orc.dense_layer(x, orc.dense_gate_matrix(out["routing"], 6), w13, w2)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


def test_layer_matches_dense_on_tiny_fp32_workload():
    cfg = mi.CONFIGS["tiny_fp32"]
    inp = mi.make(cfg)
    out = orc.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K)
    ref = orc.dense_layer(inp["x"], orc.dense_gate_matrix(out["routing"], cfg.E), inp["w13"], inp["w2"])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-10, atol=1e-12)
    assert out["routing"].counts.sum() == cfg.T * cfg.K


@pytest.mark.parametrize("name", ["mixtral", "fine_grained", "dsv3_share"])
def test_layer_matches_dense_masked_evaluation_at_workload_widths(name):
    """The per-expert loop against every expert on every token at the real widths, router
    recipes and score functions of the three bf16 workloads (64 tokens each): softmax with
    near-uniform load, softmax with a N(0,1) per-expert bias over 128 experts, sigmoid with
    Zipf-like rank offsets and four masked experts at d = 7168."""
    cfg = mi.CONFIGS[name]
    inp = mi.make(cfg, rows=64)
    out = orc.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm)
    r = out["routing"]
    assert r.counts.sum() == 64 * cfg.K
    if name == "dsv3_share":
        assert np.all(r.counts[~np.isfinite(inp["bias"])] == 0)
    ref = orc.dense_layer(inp["x"], orc.dense_gate_matrix(r, cfg.E), inp["w13"], inp["w2"])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def _rows_case(bf16):
    if bf16:
        cfg = mi.MoEConfig("rows_skew", seed=51, T=90, d=64, E=6, K=3, F=40, bf16=True, wr_std=0.3,
                           bias="normal", dy_seed=52)
    else:
        cfg = mi.CONFIGS["tiny_fp32"]
    inp = mi.make(cfg)
    dy = mi.upstream_grad(cfg)
    fwd = orc.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm)
    return cfg, inp, dy, fwd


@pytest.mark.parametrize("bf16", [False, True])
def test_single_rows_and_entries_equal_the_whole_layer(bf16):
    """layer_rows / backward_rows / wgrad_entries (the oracle's per-row and per-entry forms used
    on full-size layers) reproduce the whole-layer forward and backward, which the dense masked
    evaluation and central differences pin."""
    cfg, inp, dy, fwd = _rows_case(bf16)
    bwd = orc.backward(dy, fwd, inp["w13"], inp["w2"], cfg.K)
    r = fwd["routing"]
    M = cfg.T * cfg.K
    rows = np.random.default_rng(3).permutation(M)
    fr = orc.layer_rows(inp["x"], inp["w13"], inp["w2"], r, rows, cfg.K)
    assert np.array_equal(fr["x_perm"], fwd["x_perm"][rows])
    for k in ("pre", "h", "y_perm"):
        np.testing.assert_allclose(fr[k], fwd[k][rows], rtol=1e-12, atol=1e-13)
    br = orc.backward_rows(inp["x"], dy, inp["w13"], inp["w2"], r, rows, cfg.K)
    for k in ("dy_perm", "d_pre", "dx_perm"):
        np.testing.assert_allclose(br[k], bwd[k][rows], rtol=1e-12, atol=1e-13)
    assert np.array_equal(orc.group_of_rows(r, np.arange(M)), np.repeat(np.arange(cfg.E), r.counts))
    rng = np.random.default_rng(4)
    for e in range(cfg.E):
        n2, k2 = rng.choice(cfg.d, 5, replace=False), rng.choice(cfg.F, 7, replace=False)
        n13, k13 = rng.choice(2 * cfg.F, 9, replace=False), rng.choice(cfg.d, 4, replace=False)
        got2 = orc.wgrad_entries(inp["x"], dy, inp["w13"], inp["w2"], r, cfg.K, e, "w2", n2, k2)
        got13 = orc.wgrad_entries(inp["x"], dy, inp["w13"], inp["w2"], r, cfg.K, e, "w13", n13, k13)
        np.testing.assert_allclose(got2, bwd["dw2"][e][np.ix_(n2, k2)], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(got13, bwd["dw13"][e][np.ix_(n13, k13)], rtol=1e-11, atol=1e-13)
        if r.counts[e] == 0:
            assert not np.any(got2) and not np.any(got13)


def test_capacity_contrast():
    x, wr, w13, w2, _ = _tiny(T=60)
    out = orc.forward(x, wr, None, w13, w2, K=2)
    r = out["routing"]
    big = int(r.counts.max())
    np.testing.assert_allclose(orc.capacity_layer(x, r, w13, w2, big), out["y"], rtol=1e-11, atol=1e-12)
    dropped = orc.capacity_layer(x, r, w13, w2, big - 2)
    assert np.abs(dropped - out["y"]).max() > 1e-3


def test_router_logits_on_basis_vectors():
    rng = np.random.default_rng(19)
    wr = rng.standard_normal((5, 7)).astype(np.float32)
    x = np.eye(7, dtype=np.float32)
    np.testing.assert_array_equal(orc.router_logits(x, wr), wr.T)
    x2 = np.zeros((1, 7), np.float32)
    x2[0, 2], x2[0, 4] = 2.0, -0.5
    np.testing.assert_allclose(orc.router_logits(x2, wr)[0], 2 * wr[:, 2] - 0.5 * wr[:, 4], rtol=1e-6)


# ---------------------------------------------------------------- backward

def _fixed_route_loss(x, w13, w2, gm, dy):
    return float((dy * orc.dense_layer(x, gm, w13, w2)).sum())


def test_backward_matches_central_differences():
    T, d, E, K, F = 6, 5, 3, 2, 4
    rng = np.random.default_rng(21)
    x = rng.standard_normal((T, d))
    w13 = rng.standard_normal((E, 2 * F, d)) / math.sqrt(d)
    w2 = rng.standard_normal((E, d, F)) / math.sqrt(F)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dy = rng.standard_normal((T, d))
    fwd = orc.forward(x, None, None, w13, w2, K, logits=logits)
    bwd = orc.backward(dy, fwd, w13, w2, K)
    r = fwd["routing"]
    gm = orc.dense_gate_matrix(r, E)
    eps = 1e-6

    def fd(arr, fn):
        g = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + eps
            lp = fn()
            arr[i] = old - eps
            lm = fn()
            arr[i] = old
            g[i] = (lp - lm) / (2 * eps)
        return g

    loss = lambda: _fixed_route_loss(x, w13, w2, gm, dy)  # noqa: E731
    np.testing.assert_allclose(bwd["dx"], fd(x, loss), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(bwd["dw13"], fd(w13, loss), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(bwd["dw2"], fd(w2, loss), rtol=1e-6, atol=1e-8)
    # d_gates: derivative of the loss with respect to each slot's gate value
    dg = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            e = r.idx[t, k]
            old = gm[t, e]
            gm[t, e] = old + eps
            lp = loss()
            gm[t, e] = old - eps
            lm = loss()
            gm[t, e] = old
            dg[t, k] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(bwd["d_gates"], dg, rtol=1e-6, atol=1e-8)


def _top_k(keys_row, K):
    return [int(e) for e in sorted(range(len(keys_row)), key=lambda e: (-keys_row[e], e))[:K]]


@pytest.mark.parametrize("score", [orc.SCORE_SOFTMAX, orc.SCORE_SIGMOID])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_backward_matches_central_differences(score, renorm):
    """d_logits against central differences of the forward's own gate function, the choice held fixed."""
    T, E, K = 5, 7, 3
    rng = np.random.default_rng(40 + 2 * score + renorm)
    keys = rng.standard_normal((T, E)) * 1.5
    idx = np.array([_top_k(keys[t], K) for t in range(T)], np.int32)
    dg = rng.standard_normal((T, K))
    got = orc.route_backward(keys, idx, dg, score, renorm)
    eps = 1e-6
    fd = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            kp, km = keys[t].copy(), keys[t].copy()
            kp[e] += eps
            km[e] -= eps
            lp = np.dot(dg[t], orc.gates_from_keys(kp, idx[t], score, renorm))
            lm = np.dot(dg[t], orc.gates_from_keys(km, idx[t], score, renorm))
            fd[t, e] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-9)


def test_route_backward_closed_forms_and_invariants():
    T, E, K = 9, 6, 2
    rng = np.random.default_rng(44)
    keys = rng.standard_normal((T, E))
    idx = np.array([_top_k(keys[t], K) for t in range(T)], np.int32)
    dg = rng.standard_normal((T, K))
    unchosen = np.ones((T, E), bool)
    for t in range(T):
        unchosen[t, idx[t]] = False
    # softmax, renormalised: the gates are a softmax over the chosen keys, so
    # d key_k = g_k (dg_k - sum_j g_j dg_j) on the chosen experts and 0 elsewhere
    d = orc.route_backward(keys, idx, dg, orc.SCORE_SOFTMAX, True)
    for t in range(T):
        g = softmax(keys[t, idx[t]])
        np.testing.assert_allclose(d[t, idx[t]], g * (dg[t] - np.dot(g, dg[t])), rtol=1e-12, atol=1e-14)
    assert np.all(np.abs(d[unchosen]) < 1e-15)   # s_e * (0 - sum_j s_j ds_j), a sum that is 0 exactly
    # any softmax: adding one constant to every key changes no gate, so each row sums to 0
    for renorm in (True, False):
        d = orc.route_backward(keys, idx, dg, orc.SCORE_SOFTMAX, renorm)
        np.testing.assert_allclose(d.sum(axis=1), 0, atol=1e-13)
    # softmax without renormalisation: every expert gets a gradient
    d = orc.route_backward(keys, idx, dg, orc.SCORE_SOFTMAX, False)
    assert np.all(d[unchosen] != 0)
    # sigmoid without renormalisation: d key = dg sigma (1 - sigma) on the chosen experts
    d = orc.route_backward(keys, idx, dg, orc.SCORE_SIGMOID, False)
    for t in range(T):
        sg = expit(keys[t, idx[t]])
        np.testing.assert_allclose(d[t, idx[t]], dg[t] * sg * (1 - sg), rtol=1e-12)
    assert np.all(d[unchosen] == 0)
    # sigmoid, renormalised: scaling every chosen score by one factor leaves the gates alone,
    # so sum_k d key_k / (1 - sigma_k) = 0; unchosen experts get 0
    d = orc.route_backward(keys, idx, dg, orc.SCORE_SIGMOID, True)
    for t in range(T):
        sg = expit(keys[t, idx[t]])
        assert abs(np.sum(d[t, idx[t]] / (1 - sg))) < 1e-12
    assert np.all(d[unchosen] == 0)
    # K = 1 with renormalisation: the gate is exactly 1, so nothing flows back
    idx1 = np.array([_top_k(keys[t], 1) for t in range(T)], np.int32)
    for score in (orc.SCORE_SOFTMAX, orc.SCORE_SIGMOID):
        assert np.all(orc.route_backward(keys, idx1, dg[:, :1], score, True) == 0)


def test_router_backward_adjoint_identity_and_basis_rows():
    """<d_logits, x Wr^T> = <dWr, Wr> = <dx, x>: the backward is the adjoint of the product."""
    T, d, E = 11, 9, 4
    rng = np.random.default_rng(46)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d))
    dl = rng.standard_normal((T, E))
    dw, dx = orc.router_backward(dl, x, w)
    assert dw.shape == (E, d) and dx.shape == (T, d)
    ref = np.sum(dl * (x @ w.T))
    np.testing.assert_allclose(np.sum(dw * w), ref, rtol=1e-12)
    np.testing.assert_allclose(np.sum(dx * x), ref, rtol=1e-12)
    # x = unit row j: dWr[:, j] is that token's d_logits; Wr = unit row: dx gets d_logits column e
    xb = np.zeros((1, d))
    xb[0, 3] = 1.0
    dw1, _ = orc.router_backward(dl[:1], xb, w)
    np.testing.assert_array_equal(dw1[:, 3], dl[0])
    assert np.all(np.delete(dw1, 3, axis=1) == 0)
    wb = np.zeros((E, d))
    wb[2, 5] = 1.0
    _, dx1 = orc.router_backward(dl, x, wb)
    np.testing.assert_array_equal(dx1[:, 5], dl[:, 2])


def test_router_chain_matches_central_differences():
    """d gates -> d logits -> (dWr, dx) against differences of the fp64 router and gates."""
    T, d, E, K = 4, 6, 5, 2
    rng = np.random.default_rng(48)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d)) / math.sqrt(d)
    idx = np.array([_top_k(x[t] @ w.T, K) for t in range(T)], np.int32)
    dg = rng.standard_normal((T, K))
    for score, renorm in ((orc.SCORE_SOFTMAX, True), (orc.SCORE_SIGMOID, False)):
        def loss():
            keys = x @ w.T
            return sum(np.dot(dg[t], orc.gates_from_keys(keys[t], idx[t], score, renorm)) for t in range(T))
        dl = orc.route_backward(x @ w.T, idx, dg, score, renorm)
        dw, dx = orc.router_backward(dl, x, w)
        eps = 1e-6
        for arr, got in ((w, dw), (x, dx)):
            fd = np.zeros_like(arr)
            for i in np.ndindex(arr.shape):
                old = arr[i]
                arr[i] = old + eps
                lp = loss()
                arr[i] = old - eps
                lm = loss()
                arr[i] = old
                fd[i] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-9)


def test_backward_empty_expert_gets_zero_weight_gradient():
    T, d, E, K, F = 12, 4, 4, 2, 3
    rng = np.random.default_rng(22)
    x = rng.standard_normal((T, d))
    w13 = rng.standard_normal((E, 2 * F, d))
    w2 = rng.standard_normal((E, d, F))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 3] = -np.inf
    fwd = orc.forward(x, None, None, w13, w2, K, logits=logits)
    bwd = orc.backward(rng.standard_normal((T, d)), fwd, w13, w2, K)
    assert fwd["routing"].counts[3] == 0
    np.testing.assert_array_equal(bwd["dw13"][3], 0.0)
    np.testing.assert_array_equal(bwd["dw2"][3], 0.0)


# ---------------------------------------------------------------- workloads

def test_workload_loads_have_the_documented_shape():
    """Realised loads on token prefixes: near-uniform (Mixtral-shaped), skewed
    with empty experts (many small experts), 4 empty experts (DeepSeek-V3 share)."""
    c2 = mi.CONFIGS["mixtral"]
    i2 = mi.make(c2, rows=2048, weights=False)
    r2 = orc.route(orc.router_logits(i2["x"], i2["w_router"]), i2["bias"], c2.K)
    assert r2.counts.min() > 0.8 * 2048 * 2 / 8 and r2.counts.max() < 1.2 * 2048 * 2 / 8

    c4 = mi.CONFIGS["dsv3_share"]
    i4 = mi.make(c4, rows=1024, weights=False)
    r4 = orc.route(orc.router_logits(i4["x"], i4["w_router"]), i4["bias"], c4.K, orc.SCORE_SIGMOID)
    assert (r4.counts == 0).sum() == 4
    assert r4.counts.max() > 5 * np.median(r4.counts[r4.counts > 0]) / 2

    c5 = mi.CONFIGS["mixtral_bwd_skew"]
    hot, dead = mi.skew_choice(c5)
    lg = mi.skew_logits(orc.router_logits(i2["x"], i2["w_router"]), hot, dead)
    r5 = orc.route(lg, None, c5.K)
    assert r5.counts[hot] == 2048 and all(r5.counts[e] == 0 for e in dead)


def test_input_prefix_rows_are_reproducible():
    c = mi.CONFIGS["fine_grained"]
    a = mi.normal(c.seed, mi.TAG_X, (c.T, c.d), 1.0, True, rows=3000)
    b = mi.normal(c.seed, mi.TAG_X, (c.T, c.d), 1.0, True, rows=100)
    assert np.array_equal(a[:100], b)


# ----------------------------------------------------------------------------
# MXFP8 (OCP MX: 32-element blocks, E8M0 scales, E4M3 elements)

def test_e4m3_code_table_closed_forms():
    vals = [orc.e4m3_decode(c) for c in range(0x7F)]         # the finite positive codes
    assert vals[0] == 0.0 and vals[0x01] == 2.0 ** -9 and vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x38] == 1.0 and vals[0x7E] == 448.0
    assert all(b > a for a, b in zip(vals, vals[1:]))          # strictly increasing
    assert math.isnan(orc.e4m3_decode(0x7F)) and math.isnan(orc.e4m3_decode(0xFF))
    for c in range(0x7F):
        assert orc.e4m3_decode(c | 0x80) == -vals[c] or (c == 0 and orc.e4m3_decode(0x80) == 0.0)


def test_e4m3_encode_round_trips_ties_to_even_and_saturates():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c
    # every midpoint between neighbouring codes goes to the code with the even mantissa
    for c in range(0x7E):
        lo, hi = orc.e4m3_decode(c), orc.e4m3_decode(c + 1)
        mid = (lo + hi) / 2
        want = c if (c & 1) == 0 else c + 1
        assert orc.e4m3_encode(mid) == want, hex(c)
        assert orc.e4m3_encode(-mid) == 0x80 | want
        assert orc.e4m3_encode(lo + (hi - lo) / 4) == c and orc.e4m3_encode(hi - (hi - lo) / 4) == c + 1
    for big in (448.0, 460.0, 464.0, 479.0, 1e6):
        assert orc.e4m3_encode(big) == 0x7E and orc.e4m3_encode(-big) == 0xFE


def test_mx_quantize_scale_rule_and_error_bound():
    rng = np.random.default_rng(60)
    a = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    a[2, 32:64] = 0.0                                           # a block of zeros
    a[3, 0] = -0.0
    codes, scales = orc.mx_quantize(a)
    assert codes.shape == a.shape and scales.shape == (6, 4)
    assert scales[2, 1] == 0 and np.all(codes[2, 32:64] == 0)
    back = orc.mx_dequantize(codes, scales)
    for r in range(6):
        for b in range(4):
            blk = a[r, b * 32:(b + 1) * 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            shared = int(scales[r, b]) - 127
            assert shared == math.floor(math.log2(amax)) - 8      # the largest element lands in [256, 512)
            x = 2.0 ** shared
            err = np.abs(back[r, b * 32:(b + 1) * 32] - blk)
            # half a step of each element's binade (steps of 2^-9 x below 2^-6 x), or the saturation
            # of values above 448 x
            step = np.where(np.abs(blk) < 2.0 ** -6 * x, 2.0 ** -9 * x,
                            np.exp2(np.floor(np.log2(np.maximum(np.abs(blk), 1e-300)))) / 8)
            ok = (err <= step / 2 * (1 + 1e-12)) | ((np.abs(blk) > 448 * x) & (np.abs(back[r, b * 32:(b + 1) * 32]) == 448 * x))
            assert np.all(ok), (r, b)


def test_mx_grouped_gemm_is_exact_on_representable_values():
    """Values that E4M3 holds exactly under their block scale quantise losslessly, so the MX
    grouped GEMM equals the plain grouped GEMM of the inputs."""
    rng = np.random.default_rng(61)
    M, N, K, G = 40, 24, 64, 3
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, -1.0, -2.5, 0.25])
    a = rng.choice(grid, (M, K))
    b = rng.choice(grid, (G, N, K))
    a[:, ::32] = 3.0                                            # every block's max is 3: scale 2^-7
    b[:, :, ::32] = -3.0
    offsets = np.array([0, 10, 10, M])
    ac, asc = orc.mx_quantize(a)
    bc, bsc = orc.mx_quantize(b.reshape(G * N, K))
    np.testing.assert_array_equal(orc.mx_dequantize(ac, asc), a)
    got = orc.grouped_gemm_mx(ac, asc, bc.reshape(G, N, K), bsc.reshape(G, N, K // 32), offsets)
    np.testing.assert_array_equal(got, orc.grouped_gemm(a, b, offsets, "nk"))
