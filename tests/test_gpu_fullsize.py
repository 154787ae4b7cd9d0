"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot form these layers whole, so it checks what it can compute one
row or one entry at a time, and the GPU outputs are made complete first:

* every output buffer is filled with NaN (integers with -7) before the call, and
  afterwards no element of it may still hold the fill, so a row or tile that the
  kernels never wrote fails;
* the whole routing (indices, counts, offsets, positions, permutation) is
  compared bit for bit;
* the forward runs as the benchmark times it (the permute folded into the
  gate/up GEMM's row loads), then once more writing the permuted copy, whose
  rows must be their tokens' rows byte for byte and whose outputs must equal
  the folded forward's bit for bit;
* in every expert group, every 256-row tile and every 32-row block inside it
  (the row extent of one matrix-core fragment) contributes one seeded random row,
  so the tiles that only full sizes create (a grid dealt over the XCDs, the
  split tail of the last round) are all reached; each row of h, y_perm (and, in
  the backward, dy_perm, d_pre and dx_perm) is compared with the oracle's row
  per row (relative error 2e-2), per 32-column block (5e-2) and per element;
* y, dx and d_gates are compared on a seeded sample of tokens;
* the layer's own weight gradients are compared, for every non-empty expert,
  on one entry in every 256 x 256 output tile.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as orc
from tests.gpu_util import GATE_ATOL, TOL_BF16, by_expert, dev, f64, host

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("dropless_mixture_experts_amd")

TILE, FRAG = 256, 32
TOL_BLOCK = 5e-2    # relative error of one 32-column block of a row
TOL_ELEM_REL = 2.0 ** -7
TOL_ELEM_RMS = 3e-2


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


def tile_rows(offsets, seed):
    """One random row in every 32-row block of every 256-row tile of every group."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for t0 in range(lo, hi, TILE):
            for b0 in range(t0, min(t0 + TILE, hi), FRAG):
                rows.append(int(rng.integers(b0, min(b0 + FRAG, hi))))
    return np.array(rows, np.int64)


def poison(*tensors):
    for t in tensors:
        if t is None:
            continue
        if t.dtype in (torch.int32, torch.int64):
            t.fill_(-7)
        else:
            t.fill_(float("nan"))


def assert_written(**tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        if t.dtype in (torch.int32, torch.int64):
            assert not torch.any(t == -7).item(), f"{name}: elements left unwritten"
        else:
            assert not torch.any(torch.isnan(t)).item(), f"{name}: elements left unwritten (NaN fill)"


def rows_of(t, rows):
    return f64(t[torch.as_tensor(rows, device=t.device)])


def check_rows(what, got, ref, rows=None, offsets=None, elem=(TOL_ELEM_REL, TOL_ELEM_RMS)):
    """Row-wise, 32-column-block-wise and element-wise bounds of got against ref (fp64); the
    element bound is elem[0] |ref| + elem[1] rms(row)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n, w = ref.shape
    diff = got - ref
    den = np.linalg.norm(ref, axis=1)
    rel = np.linalg.norm(diff, axis=1) / np.where(den > 0, den, 1.0)
    where = ""
    if rows is not None:
        i = int(np.argmax(rel))
        where = f" (worst row {rows[i]}"
        if offsets is not None:
            e = int(np.searchsorted(offsets, rows[i], side="right") - 1)
            where += f", group {e}, tile {(rows[i] - offsets[e]) // TILE}"
        where += ")"
    assert np.all(rel <= TOL_BF16), f"{what}: row relative error {rel.max():.3e}{where}"
    nb = w // FRAG
    if nb > 0:
        db = np.linalg.norm(diff[:, :nb * FRAG].reshape(n, nb, FRAG), axis=2)
        rb = np.linalg.norm(ref[:, :nb * FRAG].reshape(n, nb, FRAG), axis=2)
        assert np.all(db <= TOL_BLOCK * rb), f"{what}: 32-column block error {(db / rb).max():.3e}"
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    bound = elem[0] * np.abs(ref) + elem[1] * rms
    assert np.all(np.abs(diff) <= bound), f"{what}: element error {(np.abs(diff) / bound).max():.3e} of its bound"


def _inputs(cfg):
    inp = mi.make(cfg)
    return inp, {k: dev(v) for k, v in inp.items()}


def _forward_full(cfg, inp, dv, logits, backward=False, fuse_permute=None):
    bufs = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, torch.bfloat16, backward=backward,
                          fuse_permute=fuse_permute)
    poison(bufs.topk_idx, bufs.gates, bufs.counts, bufs.offsets, bufs.slot_pos, bufs.row_src,
           bufs.x_perm, bufs.h, bufs.pre, bufs.y_perm, bufs.y)
    print(f"[fullsize] {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} K={cfg.K} F={cfg.F} "
          f"fused permute={bufs.fuse_permute}", flush=True)
    moe.layer_forward(dv["x"], dv["w_router"], dv["bias"], dv["w13"], dv["w2"], cfg.K, cfg.score, cfg.renorm,
                      bufs, logits=dev(logits))
    torch.cuda.synchronize()
    assert_written(topk_idx=bufs.topk_idx, gates=bufs.gates, counts=bufs.counts, offsets=bufs.offsets,
                   slot_pos=bufs.slot_pos, row_src=bufs.row_src, x_perm=bufs.x_perm, h=bufs.h, pre=bufs.pre,
                   y_perm=bufs.y_perm, y=bufs.y)
    return bufs


def _check_routing(bufs, r, cfg):
    np.testing.assert_array_equal(host(bufs.topk_idx), r.idx)
    np.testing.assert_array_equal(host(bufs.counts), r.counts)
    np.testing.assert_array_equal(host(bufs.offsets), r.offsets)
    np.testing.assert_array_equal(host(bufs.slot_pos), r.slot_pos)
    np.testing.assert_array_equal(host(bufs.row_src), r.row_src)
    np.testing.assert_allclose(host(bufs.gates), r.gates, atol=GATE_ATOL, rtol=0)


@pytest.mark.parametrize("name", ["mixtral", "fine_grained", "dsv3_share"])
def test_full_forward(name):
    cfg = mi.CONFIGS[name]
    inp, dv = _inputs(cfg)
    logits = orc.router_logits(inp["x"], inp["w_router"])
    bufs = _forward_full(cfg, inp, dv, logits)

    # the whole routing, bit for bit
    r = orc.route(logits, inp["bias"], cfg.K, cfg.score, cfg.renorm)
    _check_routing(bufs, r, cfg)
    if name == "dsv3_share":
        assert (r.counts == 0).sum() == 4

    # the benchmark's forward folds the permute into the gate/up GEMM: no permuted copy
    assert bufs.fuse_permute and bufs.x_perm is None

    # one row in every 32-row block of every tile of every group, against the oracle's rows
    rows = tile_rows(r.offsets, seed=7)
    ref = orc.layer_rows(inp["x"], inp["w13"], inp["w2"], r, rows, cfg.K)
    print(f"[fullsize] {name}: {len(rows)} rows checked", flush=True)
    check_rows("h", rows_of(bufs.h, rows), ref["h"], rows, r.offsets)
    check_rows("y_perm", rows_of(bufs.y_perm, rows), ref["y_perm"], rows, r.offsets)

    # the combined output of sampled tokens (a token depends only on its own row and the weights)
    S = _sample(cfg.T, 64, 8)
    fwd = orc.forward(inp["x"][S], None, inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm,
                      logits=logits[S])
    check_rows("y", f64(bufs.y)[S], fwd["y"], S)

    # the forward that writes the permuted copy: every permuted row is its token's row byte
    # for byte, and every output equals the folded forward's bit for bit
    plain = _forward_full(cfg, inp, dv, logits, fuse_permute=False)
    src = torch.as_tensor(r.row_src // cfg.K, device="cuda")
    assert torch.equal(plain.x_perm.view(torch.int16), dv["x"].view(torch.int16)[src])
    assert np.array_equal(host(plain.x_perm[torch.as_tensor(rows, device="cuda")]), ref["x_perm"])
    for n in ("h", "y_perm", "y"):
        assert torch.equal(getattr(plain, n), getattr(bufs, n)), n


@pytest.mark.parametrize("name", ["mixtral", "fine_grained", "dsv3_share"])
def test_full_fused_router(name):
    """The fused router (product and routing in one call, the benchmark's and the layer's default)
    equals the router product followed by moe_route bit for bit on every output, and routes every
    token whose top-K choice has a clear margin in the oracle's own logits as the oracle does."""
    cfg = mi.CONFIGS[name]
    inp = mi.make(cfg, weights=False)
    x, w, b = dev(inp["x"]), dev(inp["w_router"]), dev(inp["bias"])
    T, E, K = cfg.T, cfg.E, cfg.K
    i32 = dict(dtype=torch.int32, device="cuda")

    def outs():
        o = dict(logits=torch.empty((T, E), dtype=torch.float32, device="cuda"), idx=torch.empty((T, K), **i32),
                 gate=torch.empty((T, K), dtype=torch.float32, device="cuda"), counts=torch.empty((E,), **i32),
                 offs=torch.empty((E + 1,), **i32), pos=torch.empty((T * K,), **i32),
                 src=torch.empty((T * K,), **i32))
        poison(*o.values())
        return o
    a, u = outs(), outs()
    ws_a = torch.empty((max(256, moe.moe_router_route_workspace_size(T, E)),), dtype=torch.uint8, device="cuda")
    ws_u = torch.empty((max(256, moe.moe_route_workspace_size(T, E)),), dtype=torch.uint8, device="cuda")
    print(f"[fullsize] fused router {name}: T={T} d={cfg.d} E={E} K={K}", flush=True)
    moe.moe_router_route(x, w, b, K, cfg.score, cfg.renorm, a["logits"], a["idx"], a["gate"], a["counts"],
                         a["offs"], a["pos"], a["src"], ws_a)
    moe.moe_router_logits(x, w, u["logits"])
    moe.moe_route(u["logits"], b, K, cfg.score, cfg.renorm, u["idx"], u["gate"], u["counts"], u["offs"], u["pos"],
                  u["src"], ws_u)
    torch.cuda.synchronize()
    assert_written(**a)
    for k in a:
        assert torch.equal(a[k], u[k]), k
    # the permutation is a bijection that lists each group's slots in ascending order
    assert torch.equal(torch.sort(a["src"].long()).values, torch.arange(T * K, device="cuda"))
    assert torch.equal(a["src"].long()[a["pos"].long()], torch.arange(T * K, device="cuda"))
    assert int(a["counts"].sum().item()) == T * K

    logits = orc.router_logits(inp["x"], inp["w_router"])
    keys = logits.astype(np.float64) + (inp["bias"].astype(np.float64) if inp["bias"] is not None else 0.0)
    srt = -np.sort(-keys, axis=1)
    clear = (srt[:, K - 1] - srt[:, K]) > 1e-3
    assert clear.mean() > 0.9
    S = np.nonzero(clear)[0]
    r = orc.route(logits[S], inp["bias"], K, cfg.score, cfg.renorm)
    # two chosen experts closer than the product's rounding may trade places: compare the sets
    gi, gg = by_expert(host(a["idx"])[S], host(a["gate"])[S])
    ri, rg = by_expert(r.idx, r.gates)
    np.testing.assert_array_equal(gi, ri)
    np.testing.assert_allclose(gg, rg, atol=1e-4, rtol=0)
    scale = np.abs(orc.to_f64(inp["x"][S])) @ np.abs(orc.to_f64(inp["w_router"])).T
    assert np.all(np.abs(host(a["logits"])[S].astype(np.float64) - logits[S]) <= 1e-5 * scale + 1e-30)


def _tile_grid(n, rng):
    """One random index in every 256-wide tile of [0, n)."""
    return np.array([int(rng.integers(t, min(t + TILE, n))) for t in range(0, n, TILE)], np.int64)


def test_full_backward_adversarial_skew():
    """Backward of the Mixtral-shaped layer with one expert taking half of the slots and two
    experts none: every tile of the dgrad outputs and of both weight gradients."""
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    inp, dv = _inputs(cfg)
    hot, dead = mi.skew_choice(cfg)
    logits = mi.skew_logits(orc.router_logits(inp["x"], inp["w_router"]), hot, dead)
    bufs = _forward_full(cfg, inp, dv, logits, backward=True)
    dy = mi.upstream_grad(cfg)
    poison(bufs.dy_perm, bufs.d_gates, bufs.d_pre, bufs.dx_perm, bufs.dx, bufs.dw13, bufs.dw2)
    moe.layer_backward(dev(dy), dv["w13"], dv["w2"], cfg.K, bufs)
    torch.cuda.synchronize()
    assert_written(dy_perm=bufs.dy_perm, d_gates=bufs.d_gates, d_pre=bufs.d_pre, dx_perm=bufs.dx_perm,
                   dx=bufs.dx, dw13=bufs.dw13, dw2=bufs.dw2)

    r = orc.route(logits, None, cfg.K)
    _check_routing(bufs, r, cfg)
    assert r.counts[hot] == cfg.T and all(r.counts[e] == 0 for e in dead)
    for e in dead:
        assert not torch.any(bufs.dw13[e]).item() and not torch.any(bufs.dw2[e]).item()

    rows = tile_rows(r.offsets, seed=9)
    print(f"[fullsize] backward: {len(rows)} rows checked", flush=True)
    ref = orc.backward_rows(inp["x"], dy, inp["w13"], inp["w2"], r, rows, cfg.K)
    check_rows("dy_perm", rows_of(bufs.dy_perm, rows), ref["dy_perm"], rows, r.offsets)
    # dG = dH U silu'(G): dH carries an absolute error (an fp32 sum of bf16-rounded terms) that
    # the heavy-tailed factor U silu'(G) multiplies, so single elements reach a few percent of
    # the row's rms where |U silu'(G)| is large; rows and 32-column blocks keep the tight bars
    check_rows("d_pre", rows_of(bufs.d_pre, rows), ref["d_pre"], rows, r.offsets, elem=(2.0 ** -6, 0.1))
    check_rows("dx_perm", rows_of(bufs.dx_perm, rows), ref["dx_perm"], rows, r.offsets)

    S = _sample(cfg.T, 64, 11)
    fwd = orc.forward(inp["x"][S], None, None, inp["w13"], inp["w2"], cfg.K, logits=logits[S])
    bwd = orc.backward(dy[S], fwd, inp["w13"], inp["w2"], cfg.K)
    check_rows("y", f64(bufs.y)[S], fwd["y"], S)
    check_rows("dx", f64(bufs.dx)[S], bwd["dx"], S)
    dg = host(bufs.d_gates)[S].astype(np.float64)
    assert np.linalg.norm(dg - bwd["d_gates"]) <= TOL_BF16 * np.linalg.norm(bwd["d_gates"])

    # the layer's own weight gradients: one entry in every 256 x 256 output tile of each expert
    rng = np.random.default_rng(12)
    for e in range(cfg.E):
        if r.counts[e] == 0:
            continue
        for which, dw, N, Kd in (("w2", bufs.dw2, cfg.d, cfg.F), ("w13", bufs.dw13, 2 * cfg.F, cfg.d)):
            n_idx, k_idx = _tile_grid(N, rng), _tile_grid(Kd, rng)
            want = orc.wgrad_entries(inp["x"], dy, inp["w13"], inp["w2"], r, cfg.K, e, which, n_idx, k_idx)
            got = dw[e][torch.as_tensor(n_idx, device="cuda")][:, torch.as_tensor(k_idx, device="cuda")]
            got = host(got).astype(np.float64)
            err = np.abs(got - want)
            rms = np.sqrt(np.mean(want * want))
            assert np.linalg.norm(err) <= TOL_BF16 * np.linalg.norm(want), (which, e)
            assert np.all(err <= 0.1 * rms), (which, e, float(err.max() / rms))
