"""Benchmark of the dropless MoE layer forward on one MI355X.

One step = the whole forward hot path over one batch of synthetic tokens:
router logits -> top-K routing (histogram, offsets, stable positions) ->
permute -> grouped GEMM gate/up + SwiGLU -> grouped GEMM down -> combine.
Inputs and weights are resident in HBM before the timed region.

Prints ONE JSON line.  value = tokens/s of the layer forward; the roofline
object reports the dominant kernel (the gate/up grouped GEMM) against the
bf16 dense MFMA peak, with its duration measured by HIP events on the stream
the kernels run on; cpu_baseline times the CPU oracle on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (matrix)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (MX formats included)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral",
                    choices=["mixtral", "fine_grained", "dsv3_share", "tiny_fp32"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters, if present")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the adversarial-skew Mixtral-shaped workload instead "
                         "(reported as an extra line, not the headline)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="time the layer forward with MXFP8 expert GEMMs instead (weights quantised once "
                         "before the timed region, activations quantised inside every step)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain elementwise pass over 512 MiB (3 launches of torch's neg "
                         "kernel: 512 MiB read, 512 MiB written) to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


KERNEL_SOURCES = ["grouped_gemm.hip", "common.h"]


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: edits to comments leave
    the code, and so the counters taken on it, unchanged."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """sha256 of the grouped GEMM code (comments stripped): traffic figures are valid only for it."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dropless_mixture_experts_amd", "csrc", name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(cfg, inp, target_s: float) -> dict | None:
    """The CPU oracle (never tuned) on the first S tokens of the same workload."""
    if target_s <= 0:
        return None
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1

    def run(S):
        t0 = time.perf_counter()
        orc.forward(inp["x"][:S], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score,
                    cfg.renorm)
        return time.perf_counter() - t0

    # widening the weights to fp64 is a fixed cost per call, so grow the sample until the
    # run itself lasts about target_s
    S = min(64, cfg.T)
    dt = run(S)
    while dt < 0.6 * target_s and S < cfg.T:
        S = int(min(cfg.T, max(2 * S, S * 0.9 * target_s / max(dt, 1e-3))))
        dt = run(S)
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of the {cfg.name} workload, full forward "
                      f"(router, top-K, permute, per-expert fp64 GEMMs, combine) in {dt:.1f} s",
            "host": host_description(cores)}


def host_description(threads: int) -> str:
    """CPU model, logical CPUs and the BLAS the oracle's NumPy uses."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api', 'blas')} {libs[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    return f"{model}, {os.cpu_count()} logical CPUs visible, {blas} with {threads} threads"


def copy_bandwidth(torch) -> float:
    """On-box HBM reference: GB/s (bytes read + written) of a 1 GiB device copy, median of five
    launches, each after a 1 GiB elementwise pass that evicts the caches."""
    src = torch.empty(512 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    flush_a = torch.empty(256 << 20, dtype=torch.float32, device="cuda").fill_(2.0)
    flush_b = torch.empty_like(flush_a)
    ts = []
    for _ in range(6):
        torch.neg(flush_a, out=flush_b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts[1:])[2]
    del src, dst, flush_a, flush_b
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import dropless_mixture_experts_amd as moe
    import moe_inputs as mi

    if args.backward:
        return bench_backward(args, torch, moe, mi)
    if args.mxfp8:
        return bench_mxfp8(args, torch, moe, mi)
    cfg = mi.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    inp = mi.make(cfg)
    gen_s = time.perf_counter() - t_gen
    dt = torch.bfloat16 if cfg.bf16 else torch.float32
    x, wr, b = to_dev(inp["x"], torch), to_dev(inp["w_router"], torch), to_dev(inp["bias"], torch)
    w13, w2 = to_dev(inp["w13"], torch), to_dev(inp["w2"], torch)
    bufs = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, dt)
    stream = torch.cuda.current_stream()

    # bf16: the fused router (product + routing in one call); fp32: product, then routing
    fused = cfg.bf16
    names = (["router_route"] if fused else ["router", "route"]) + ["permute", "gemm_gate_up", "gemm_down", "combine"]
    nk = len(names)
    rr_ws = torch.empty((max(moe.moe_router_route_workspace_size(cfg.T, cfg.E), 256),), dtype=torch.uint8,
                        device="cuda")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        i = 0
        mark(i)
        if fused:
            moe.moe_router_route(x, wr, b, cfg.K, cfg.score, cfg.renorm, None, bufs.topk_idx, bufs.gates,
                                 bufs.counts, bufs.offsets, bufs.slot_pos, bufs.row_src, rr_ws)
        else:
            moe.moe_router_logits(x, wr, bufs.logits)
            i += 1
            mark(i)
            moe.moe_route(bufs.logits, b, cfg.K, cfg.score, cfg.renorm, bufs.topk_idx, bufs.gates, bufs.counts,
                          bufs.offsets, bufs.slot_pos, bufs.row_src, bufs.ws)
        i += 1
        mark(i)
        moe.moe_permute(x, cfg.K, bufs.slot_pos, bufs.x_perm)
        mark(i + 1)
        moe.moe_grouped_gemm(bufs.x_perm, w13, moe.MOE_LAYOUT_NK, bufs.offsets, bufs.h, moe.MOE_EPI_SWIGLU,
                             workspace=bufs.gemm_ws)
        mark(i + 2)
        moe.moe_grouped_gemm(bufs.h, w2, moe.MOE_LAYOUT_NK, bufs.offsets, bufs.y_perm, moe.MOE_EPI_NONE,
                             workspace=bufs.gemm_ws)
        mark(i + 3)
        moe.moe_unpermute_combine(bufs.y_perm, bufs.slot_pos, bufs.gates, cfg.T, cfg.K, bufs.y)
        mark(i + 4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the layer captured once as a HIP graph (group sizes stay on the device, so one capture
    # serves every routing); the timed region is K replays, one layer forward each
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)

    # per-kernel breakdown: K eager steps with HIP events on the launch stream around every call
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    per = np.zeros(len(names))
    for ev in evs:
        per += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(nk)])
    per /= max(args.steps, 1)
    kms = dict(zip(names, per.tolist()))

    M = cfg.T * cfg.K
    esz = 2 if cfg.bf16 else 4
    flops_up = 2.0 * M * (2 * cfg.F) * cfg.d
    flops_down = 2.0 * M * cfg.F * cfg.d
    peak = PEAK_BF16_TFLOPS if cfg.bf16 else PEAK_F32_TFLOPS
    tf_up = flops_up / (kms["gemm_gate_up"] * 1e-3) / 1e12
    tf_down = flops_down / (kms["gemm_down"] * 1e-3) / 1e12
    tf_gg = (flops_up + flops_down) / ((kms["gemm_gate_up"] + kms["gemm_down"]) * 1e-3) / 1e12
    perm_bytes = (cfg.T + M) * cfg.d * esz + 4 * M
    comb_bytes = (M + cfg.T) * cfg.d * esz + 8 * M
    router_bytes = cfg.T * cfg.d * esz + cfg.E * cfg.d * esz + 4 * cfg.T * cfg.E
    # fused: x and W once, then per slot the index and gate written, its in-tile rank written
    # and read back, its position and its inverse written
    router_route_bytes = cfg.T * cfg.d * esz + cfg.E * cfg.d * esz + 24 * M

    traffic = None
    try:
        with open(args.traffic) as f:
            tr = json.load(f)
        rec = tr.get(f"{cfg.name}/gemm_gate_up")
        if rec and rec.get("source_sha256") == kernel_source_hash():
            traffic = rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    counts = bufs.counts.cpu().numpy()
    # after the timed region; left out of the counter-calibration runs, whose own 512 MiB pass must
    # be the only elementwise kernel of its kind
    copy_gbs = copy_bandwidth(torch) if not args.calib_copy else float("nan")
    cpu = cpu_baseline(cfg, inp, args.cpu_seconds)
    hbm = {"permute": perm_bytes / (kms["permute"] * 1e-3) / 1e9,
           "combine": comb_bytes / (kms["combine"] * 1e-3) / 1e9,
           **({"router_route": router_route_bytes / (kms["router_route"] * 1e-3) / 1e9} if fused else
              {"router": router_bytes / (kms["router"] * 1e-3) / 1e9})}

    out = {
        "metric": "MoE layer forward tokens/s (grouped-GEMM TFLOP/s and % of bf16 MFMA peak alongside)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.bf16 else "f32",
        "data": "synthetic (seeded N(0,1) tokens, random-init router and SwiGLU experts)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.K,
                   "ffn": cfg.F, "score": "sigmoid" if cfg.score else "softmax", "renorm": cfg.renorm,
                   "parallelism": "single GPU"},
        "grouped_gemm": {"tflops": tf_gg, "frac_of_peak": tf_gg / peak, "gate_up_tflops": tf_up,
                         "down_tflops": tf_down, "flops_per_step": flops_up + flops_down},
        "kernels_ms": kms,
        "timing": {"value": "one HIP-graph replay of the layer per step",
                   "eager_ms_per_step": eager_ms_per_step,
                   "eager_tokens_per_s": cfg.T / (eager_ms_per_step * 1e-3)},
        "hbm_gbs": hbm,
        # each HBM rate as a fraction of the spec peak (8 TB/s) and of an on-box 1 GiB copy
        "hbm_frac": {k: {"of_spec": v / 8000.0, "of_onbox_copy": v / copy_gbs} for k, v in hbm.items()},
        "onbox_copy_gbs": copy_gbs,
        "load": {"min": int(counts.min()), "max": int(counts.max()), "empty": int((counts == 0).sum())},
        "roofline": {"kernel": "grouped GEMM gate/up + SwiGLU", "bound": "mfma", "achieved": tf_up,
                     "peak": peak, "unit": "TFLOP/s", "frac": tf_up / peak, "traffic": traffic},
        "cpu_baseline": cpu,
        "input_generation_s": gen_s,
    }
    print(json.dumps(out), flush=True)
    if args.calib_copy:
        # one kernel per launch that reads and writes exactly 512 MiB (a device-to-device copy may
        # be split into several dispatches)
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()


def bench_backward(args, torch, moe, mi):
    """Backward of the Mixtral-shaped layer with one expert taking half of the slots and two none:
    combine backward, SwiGLU-backward dgrad, down wgrad, gate/up dgrad, gate/up wgrad,
    permute backward, then the router's backward (d_gates -> d_logits -> dWr, and its share of
    dX); routing held fixed."""
    import oracle as orc
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    torch.cuda.set_device(0)
    inp = mi.make(cfg)
    hot, dead = mi.skew_choice(cfg)
    logits = mi.skew_logits(orc.router_logits(inp["x"], inp["w_router"]), hot, dead)
    dev = {k: to_dev(v, torch) for k, v in inp.items()}
    dy = to_dev(mi.upstream_grad(cfg), torch)
    bufs = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, torch.bfloat16, backward=True)
    moe.layer_forward(dev["x"], dev["w_router"], None, dev["w13"], dev["w2"], cfg.K, cfg.score, cfg.renorm,
                      bufs, logits=to_dev(logits, torch))
    stream = torch.cuda.current_stream()
    b = bufs
    names = ["combine_bwd", "dgrad_down_dswiglu", "wgrad_down", "dgrad_gate_up", "wgrad_gate_up", "permute_bwd",
             "route_bwd", "router_bwd"]
    nk = len(names)
    logits_dev = to_dev(logits, torch)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        moe.moe_permute(dy, cfg.K, b.slot_pos, b.dy_perm, row_scale=b.gates, y_perm_dot=b.y_perm,
                        dgate_out=b.d_gates)
        mark(1)
        moe.moe_grouped_gemm(b.dy_perm, dev["w2"], moe.MOE_LAYOUT_KN, b.offsets, b.d_pre, moe.MOE_EPI_DSWIGLU,
                             epi_in=b.pre)
        mark(2)
        moe.moe_grouped_gemm_wgrad(b.h, b.dy_perm, b.offsets, b.dw2)
        mark(3)
        moe.moe_grouped_gemm(b.d_pre, dev["w13"], moe.MOE_LAYOUT_KN, b.offsets, b.dx_perm, moe.MOE_EPI_NONE,
                             workspace=b.gemm_ws)
        mark(4)
        moe.moe_grouped_gemm_wgrad(b.x_perm, b.d_pre, b.offsets, b.dw13)
        mark(5)
        moe.moe_unpermute_combine(b.dx_perm, b.slot_pos, None, cfg.T, cfg.K, b.dx)
        mark(6)
        moe.moe_route_backward(logits_dev, None, b.topk_idx, b.d_gates, cfg.score, cfg.renorm, b.d_logits)
        mark(7)
        moe.moe_router_logits_backward(b.d_logits, dev["x"], dev["w_router"], b.dw_router, b.dx, b.rb_ws,
                                       accumulate=True)
        mark(8)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    per = np.zeros(nk)
    for ev in evs:
        per += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(nk)])
    per /= max(args.steps, 1)
    kms = dict(zip(names, per.tolist()))
    M = cfg.T * cfg.K
    fl = {"dgrad_down_dswiglu": 2.0 * M * cfg.d * cfg.F, "wgrad_down": 2.0 * M * cfg.d * cfg.F,
          "dgrad_gate_up": 2.0 * M * 2 * cfg.F * cfg.d, "wgrad_gate_up": 2.0 * M * 2 * cfg.F * cfg.d}
    tf = {k: fl[k] / (kms[k] * 1e-3) / 1e12 for k in fl}
    total_fl = sum(fl.values())
    out = {"metric": "MoE layer backward tokens/s (routing held fixed)", "value": cfg.T / (ms * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.K,
                      "ffn": cfg.F, "hot_expert_slots": int(bufs.counts.max().item()),
                      "empty_experts": int((bufs.counts == 0).sum().item())},
           "gemm_tflops": tf, "gemm_total_tflops": total_fl / (sum(kms[k] for k in fl) * 1e-3) / 1e12,
           "kernels_ms": kms,
           # router backward bytes: the d_logits pass (logits read, d_logits written: 8 T E) and the
           # product's x read for dWr plus dX read and written for its share (3 T d b)
           "router_bwd_gbs": {"route_bwd": 8.0 * cfg.T * cfg.E / (kms["route_bwd"] * 1e-3) / 1e9,
                              "router_bwd": 3.0 * cfg.T * cfg.d * 2 / (kms["router_bwd"] * 1e-3) / 1e9}}
    print(json.dumps(out), flush=True)


def bench_mxfp8(args, torch, moe, mi):
    """The bf16 layer forward with both expert GEMMs on MXFP8 operands: the tokens (then their
    codes are permuted) and H are quantised (32-value blocks, E8M0 scales, E4M3 values) inside
    every step; the weights once, before the timed region, as stored MX weights would be."""
    cfg = mi.CONFIGS[args.workload]
    if not cfg.bf16:
        raise SystemExit("--mxfp8 needs a bf16 workload")
    torch.cuda.set_device(0)
    inp = mi.make(cfg)
    x, wr, b = to_dev(inp["x"], torch), to_dev(inp["w_router"], torch), to_dev(inp["bias"], torch)
    w13, w2 = to_dev(inp["w13"], torch), to_dev(inp["w2"], torch)
    E, d, F, K, T = cfg.E, cfg.d, cfg.F, cfg.K, cfg.T
    M = T * K
    bufs = moe.MoEBuffers(T, d, E, K, F, torch.bfloat16)
    u8 = dict(dtype=torch.uint8, device="cuda")
    w13c, w13s = torch.empty(E, 2 * F, d, **u8), torch.empty(E, 2 * F, d // 32, **u8)
    w2c, w2s = torch.empty(E, d, F, **u8), torch.empty(E, d, F // 32, **u8)
    moe.moe_mx_quantize(w13.view(E * 2 * F, d), w13c.view(E * 2 * F, d), w13s.view(E * 2 * F, d // 32))
    moe.moe_mx_quantize(w2.view(E * d, F), w2c.view(E * d, F), w2s.view(E * d, F // 32))
    del w13, w2
    tq, ts = torch.empty(T, d, **u8), torch.empty(T, d // 32, **u8)
    xq, xs = torch.empty(M, d, **u8), torch.empty(M, d // 32, **u8)
    hq, hs = torch.empty(M, F, **u8), torch.empty(M, F // 32, **u8)
    rr_ws = torch.empty((max(moe.moe_router_route_workspace_size(T, E), 256),), **u8)
    stream = torch.cuda.current_stream()
    names = ["router_route", "quantize_x", "permute", "gemm_gate_up", "quantize_h", "gemm_down", "combine"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        moe.moe_router_route(x, wr, b, K, cfg.score, cfg.renorm, None, bufs.topk_idx, bufs.gates, bufs.counts,
                             bufs.offsets, bufs.slot_pos, bufs.row_src, rr_ws)
        mark(1)
        moe.moe_mx_quantize(x, tq, ts)
        mark(2)
        moe.moe_permute_mx(tq, ts, K, bufs.slot_pos, xq, xs)
        mark(3)
        moe.moe_grouped_gemm_mx(xq, xs, w13c, w13s, bufs.offsets, bufs.h, moe.MOE_EPI_SWIGLU)
        mark(4)
        moe.moe_mx_quantize(bufs.h, hq, hs)
        mark(5)
        moe.moe_grouped_gemm_mx(hq, hs, w2c, w2s, bufs.offsets, bufs.y_perm, moe.MOE_EPI_NONE)
        mark(6)
        moe.moe_unpermute_combine(bufs.y_perm, bufs.slot_pos, bufs.gates, T, K, bufs.y)
        mark(7)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = np.zeros(len(names))
    for ev in evs:
        per += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(len(names))])
    per /= max(args.steps, 1)
    kms = dict(zip(names, per.tolist()))
    fl_up, fl_down = 2.0 * M * 2 * F * d, 2.0 * M * F * d
    tf_up = fl_up / (kms["gemm_gate_up"] * 1e-3) / 1e12
    tf_down = fl_down / (kms["gemm_down"] * 1e-3) / 1e12
    out = {"metric": "MoE layer forward tokens/s, MXFP8 expert GEMMs (weights quantised once)",
           "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp8",
           "data": "synthetic (seeded N(0,1) tokens, random-init router and SwiGLU experts)",
           "config": {"workload": cfg.name, "tokens": T, "d_model": d, "experts": E, "top_k": K, "ffn": F,
                      "parallelism": "single GPU"},
           "grouped_gemm": {"gate_up_tflops": tf_up, "down_tflops": tf_down,
                            "tflops": (fl_up + fl_down) / ((kms["gemm_gate_up"] + kms["gemm_down"]) * 1e-3) / 1e12},
           "kernels_ms": kms,
           "quantize_gbs": {"x": (T * d * 3 + T * d // 32) / (kms["quantize_x"] * 1e-3) / 1e9,
                            "h": (M * F * 3 + M * F // 32) / (kms["quantize_h"] * 1e-3) / 1e9},
           "roofline": {"kernel": "MXFP8 grouped GEMM gate/up + SwiGLU", "bound": "mfma", "achieved": tf_up,
                        "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": tf_up / PEAK_FP8_TFLOPS, "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
