"""The allocation-free fused router against the fused router with a caller workspace.

moe_router_route_noalloc keeps its per-chunk expert histograms in the library's
static device array instead of a caller workspace.  It runs the same kernels, so
every output must equal moe_router_route's bit for bit; two calls in a row, the
second on a smaller input, show that the array's leftover contents from the first
call never leak into the second.
"""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("dropless_mixture_experts_amd")

# (T, d, E, K, score, renorm, bias): a fine-grained-like routing (64-token chunks, 128 experts),
# then a smaller one (32-token chunks, 8 experts, sigmoid scores, a masked expert)
CASES = [(16384, 2048, 128, 8, 0, True, "normal"), (3000, 512, 8, 2, 1, True, "masked")]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _outs(T, E, K):
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(logits=torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda"),
                idx=torch.full((T, K), -7, **i32),
                gate=torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), -7, **i32), offs=torch.full((E + 1,), -7, **i32),
                pos=torch.full((T * K,), -7, **i32), src=torch.full((T * K,), -7, **i32))


def test_router_route_noalloc_matches_workspace_form_on_two_calls():
    for i, (T, d, E, K, score, renorm, bias_kind) in enumerate(CASES):
        print(f"[no-alloc] call {i}: T={T} d={d} E={E} K={K} score={score}", flush=True)
        rng = np.random.default_rng(900 + i)
        x = dev(mi.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)))
        w = dev(mi.f32_to_bf16_bits((rng.standard_normal((E, d)) * 1.5 / math.sqrt(d)).astype(np.float32)))
        bias = rng.standard_normal(E).astype(np.float32)
        if bias_kind == "masked":
            bias[3] = -np.inf
        b = dev(bias)
        ref, got = _outs(T, E, K), _outs(T, E, K)
        ws = torch.empty((max(256, moe.moe_router_route_workspace_size(T, E)),), dtype=torch.uint8, device="cuda")
        moe.moe_router_route(x, w, b, K, score, renorm, ref["logits"], ref["idx"], ref["gate"], ref["counts"],
                             ref["offs"], ref["pos"], ref["src"], ws)
        moe.moe_router_route_noalloc(x, w, b, K, score, renorm, got["logits"], got["idx"], got["gate"],
                                     got["counts"], got["offs"], got["pos"], got["src"])
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], got[k]), (i, k)
        assert int(got["counts"].sum().item()) == T * K
        assert not torch.any(got["src"] < 0).item()
        if bias_kind == "masked":
            assert int(got["counts"][3].item()) == 0
