"""Benchmark of the dropless MoE layer forward on one MI355X.

One step = the whole forward hot path over one batch of synthetic tokens:
router logits -> top-K routing (histogram, offsets, stable positions) ->
permute -> grouped GEMM gate/up + SwiGLU -> grouped GEMM down -> combine,
with the permute done by the gate/up GEMM's own row loads for bf16 layers
(the forward of a layer that keeps no backward buffers).
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
    ap.add_argument("--gemm-zipf", action="store_true",
                    help="time the two grouped GEMMs alone on 32768 rows in 32 groups of exact Zipf(1.2) sizes "
                         "(d = 7168, F = 2048; 4 empty groups) instead (an extra line, not the headline)")
    ap.add_argument("--cold-reps", type=int, default=100,
                    help="launches of each kernel timed alone with the caches flushed before each one")
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the GPU clock with amd-smi")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the shorter backward and MXFP8 runs that the Mixtral-shaped forward line carries "
                         "under extra_lines")
    ap.add_argument("--no-train-form", action="store_true",
                    help="skip the training form of the forward (permuted copy written, pre-activations saved)")
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


def measured_traffic(path: str, key: str):
    """Calibrated HBM bytes per launch recorded under key in the counter file at path, or None when
    absent or recorded for other GEMM code (a different kernel_source_hash())."""
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
        if rec and rec.get("source_sha256") == kernel_source_hash():
            return rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


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


def stream_rates(torch) -> dict:
    """On-box HBM references, GB/s, each the median of five launches after a read-only 1 GiB
    pass that evicts the caches: a 1 GiB device copy (bytes read + written), a read-mostly pass
    (the column sums of a [32, 8M] fp32 matrix: 1 GiB read, 32 MiB written) and a write-only
    pass over 1 GiB (a fill; the 256 MB Infinity Cache may hold part of it when the clock stops)."""
    src = torch.empty(512 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    rd = torch.ones((32, 8 << 20), dtype=torch.float32, device="cuda")
    col = torch.empty((8 << 20,), dtype=torch.float32, device="cuda")
    acc = torch.empty((), dtype=torch.float32, device="cuda")

    def med(fn):
        ts = []
        for _ in range(6):
            torch.sum(flush, dim=0, out=acc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts[1:])[2]
    gib = float(1 << 30)
    out = {"copy": 2 * gib / (med(lambda: dst.copy_(src)) * 1e-3) / 1e9,
           "read": (gib + (32 << 20)) / (med(lambda: torch.sum(rd, dim=0, out=col)) * 1e-3) / 1e9,
           "write": gib / (med(lambda: dst.fill_(0.5)) * 1e-3) / 1e9}
    del src, dst, flush, rd, col, acc
    return out


class ColdTimer:
    """Times single launches with the caches cold: before each launch a read-only pass over
    1 GiB (a sum) evicts the 4 MB L2s and the 256 MB Infinity Cache, leaving clean lines, so
    the timed kernel neither hits on its inputs nor pays for earlier dirty lines.  HIP events
    on the launch stream bracket the launch alone."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.buf = torch.ones((256 << 20,), dtype=torch.float32, device="cuda")
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def time(self, fn, reps: int) -> dict:
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            torch.sum(self.buf, dim=0, out=self.out)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        ts = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
        return {"median": float(np.median(ts)), "min": float(ts.min()), "mean": float(ts.mean()), "reps": int(reps)}


def _find_gfx_clocks(obj, out, under_gfx=False):
    """MHz values of the graphics clocks anywhere in amd-smi's JSON."""
    if isinstance(obj, dict):
        for k, v in obj.items():
            key = str(k).lower()
            gfx = under_gfx or key.startswith("gfx")
            if gfx and key == "clk":
                val = v.get("value") if isinstance(v, dict) else v
                try:
                    out.append(float(val))
                except (TypeError, ValueError):
                    pass
            else:
                _find_gfx_clocks(v, out, gfx)
    elif isinstance(obj, list):
        for v in obj:
            _find_gfx_clocks(v, out, under_gfx)


def sample_clock(torch, replay, seconds: float = 2.0) -> dict | None:
    """The graphics clock under sustained load: amd-smi sampled from a thread while the layer
    graph replays back to back."""
    import shutil
    import subprocess
    import threading
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    samples, raw = [], []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([exe, "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                raw.append(r.stdout[:400])
                vals = []
                _find_gfx_clocks(json.loads(r.stdout), vals)
                vals = [v for v in vals if v > 0]
                if vals:
                    samples.append(float(np.mean(vals)))
            except Exception:
                pass
            time.sleep(0.1)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            replay()
        n += 20
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return {"sclk_mhz_median": None, "samples": 0, "raw": raw[:1]}
    return {"sclk_mhz_median": float(np.median(samples)), "sclk_mhz_min": float(min(samples)),
            "sclk_mhz_max": float(max(samples)), "samples": len(samples), "replays": n,
            "source": "amd-smi metric -c, sampled while the layer graph replays"}


def one_core_oracle(cfg_tiny, cfg, inp) -> dict:
    """The oracle on one BLAS thread: the tiny fp32 workload (median of 5 runs) and the first
    tokens of the bf16 workload, with fp64 GFLOP/s of the expert and router products."""
    import moe_inputs as mi
    import oracle as orc
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None

    def flops(c, T):
        return T * (2.0 * c.d * c.E + c.K * 6.0 * c.d * c.F)

    out = {}
    with threadpool_limits(limits=1):
        ti = mi.make(cfg_tiny)
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            orc.forward(ti["x"], ti["w_router"], ti["bias"], ti["w13"], ti["w2"], cfg_tiny.K, cfg_tiny.score,
                        cfg_tiny.renorm)
            ts.append(time.perf_counter() - t0)
        dt = float(np.median(ts))
        out[cfg_tiny.name] = {"tokens_per_s": cfg_tiny.T / dt, "seconds": dt,
                              "gflops_fp64": flops(cfg_tiny, cfg_tiny.T) / dt / 1e9}
        S = min(128, cfg.T)
        t0 = time.perf_counter()
        orc.forward(inp["x"][:S], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.score, cfg.renorm)
        dt = time.perf_counter() - t0
        out[cfg.name] = {"tokens_per_s": S / dt, "seconds": dt, "tokens": S,
                         "gflops_fp64": flops(cfg, S) / dt / 1e9}
    out["threads"] = 1
    return out


def capture(torch, fn):
    """fn captured once as a HIP graph (after one run on a side stream, as capture requires)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def time_replays(torch, graph, warmup: int, steps: int) -> float:
    for _ in range(max(warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / max(steps, 1)


def replay_stats(torch, graph, stream, reps: int, flush=None) -> dict:
    """Each of reps graph replays bracketed by its own HIP events (flush(), when given, runs
    before each replay, outside the events): median, min and mean ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ts = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    return {"median": float(np.median(ts)), "min": float(ts.min()), "mean": float(ts.mean()), "reps": int(reps)}


def time_steps(torch, steps, stream, reps: int) -> tuple[dict, float]:
    """Average duration of each (name, call) over reps eager passes, from HIP events recorded
    on the launch stream between the calls; and the eager ms per pass."""
    n = len(steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        ev[0].record(stream)
        for i, (_, call) in enumerate(steps):
            call()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) * 1e3 / max(reps, 1)
    per = np.zeros(n)
    for ev in evs:
        per += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    per /= max(reps, 1)
    return dict(zip([nm for nm, _ in steps], per.tolist())), eager


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
        print(json.dumps(bench_backward(args, torch, moe, mi)), flush=True)
    elif args.mxfp8:
        print(json.dumps(bench_mxfp8(args, torch, moe, mi)), flush=True)
    elif args.gemm_zipf:
        bench_gemm_zipf(args, torch, moe, mi)
    else:
        out = bench_forward(args, torch, moe, mi)
        if out["config"]["workload"] == "mixtral" and not args.no_extras:
            out["extra_lines"] = extra_lines(args, torch, moe, mi)
        print(json.dumps(out), flush=True)
    if args.calib_copy:
        # one kernel per launch that reads and writes exactly 512 MiB (a device-to-device copy may
        # be split into several dispatches)
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()


def bench_forward(args, torch, moe, mi) -> dict:
    """The headline line: the layer forward of one workload (args.workload), as a dict."""
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

    # the product's forward, call for call (bf16: the fused router; fp32: product, then routing)
    steps = moe.forward_steps(x, wr, b, w13, w2, cfg.K, cfg.score, cfg.renorm, bufs)
    fused = steps[0][0] == "router_route"

    def run_all():
        for _, call in steps:
            call()

    for _ in range(args.warmup):
        run_all()
    torch.cuda.synchronize()

    # the layer captured once as a HIP graph (group sizes stay on the device, so one capture
    # serves every routing); the timed region is K replays, one layer forward each
    graph = capture(torch, run_all)
    ms_per_step = time_replays(torch, graph, args.warmup, args.steps)

    # per-kernel breakdown inside the layer: K eager passes, HIP events on the launch stream
    kms, eager_ms_per_step = time_steps(torch, steps, stream, args.steps)

    # each kernel alone with the caches flushed before every launch (median and min of the reps)
    cold = ColdTimer(torch, stream)
    kcold = {name: cold.time(call, args.cold_reps) for name, call in steps}
    # the layer replay by replay: warm (back to back) and cold (caches flushed before each)
    layer_ms = {"warm": replay_stats(torch, graph, stream, args.cold_reps),
                "cold": replay_stats(torch, graph, stream, args.cold_reps,
                                     flush=lambda: torch.sum(cold.buf, dim=0, out=cold.out))}
    if bufs.x_perm is None:
        # the layer reads token rows inside the gate/up GEMM; the standalone permute (the call
        # a training forward and other callers make) is timed on its own, cold, for its HBM rate
        xp = torch.empty((cfg.T * cfg.K, cfg.d), dtype=dt, device="cuda")
        kcold["permute"] = cold.time(lambda: moe.moe_permute(x, cfg.K, bufs.slot_pos, xp), args.cold_reps)
        del xp
    del cold
    torch.cuda.empty_cache()

    M = cfg.T * cfg.K
    esz = 2 if cfg.bf16 else 4
    flops_up = 2.0 * M * (2 * cfg.F) * cfg.d
    flops_down = 2.0 * M * cfg.F * cfg.d
    peak = PEAK_BF16_TFLOPS if cfg.bf16 else PEAK_F32_TFLOPS
    tf_up = flops_up / (kms["gemm_gate_up"] * 1e-3) / 1e12
    tf_down = flops_down / (kms["gemm_down"] * 1e-3) / 1e12
    tf_gg = (flops_up + flops_down) / ((kms["gemm_gate_up"] + kms["gemm_down"]) * 1e-3) / 1e12
    # (bytes read, bytes written) of each HBM-bound call
    nrw = {
        "permute": (cfg.T * cfg.d * esz + 4 * M, M * cfg.d * esz),
        "combine": (M * cfg.d * esz + 8 * M, cfg.T * cfg.d * esz),
        # fused: x and W once, then per slot the index and gate written, its in-tile rank written
        # and read back, its position and its inverse written, and the fp32 logits written
        "router_route": (cfg.T * cfg.d * esz + cfg.E * cfg.d * esz + 4 * M, 20 * M + 4 * cfg.T * cfg.E),
        "router": (cfg.T * cfg.d * esz + cfg.E * cfg.d * esz, 4 * cfg.T * cfg.E),
    }
    nbytes = {k: r + w for k, (r, w) in nrw.items()}

    traffic = measured_traffic(args.traffic, f"{cfg.name}/gemm_gate_up")

    tokens_per_s = cfg.T / (ms_per_step * 1e-3)

    # the training form of the forward: the permuted copy written (the weight gradient reads it)
    # and the SwiGLU pre-activations saved; graph replays as for value
    train = None
    if not args.no_train_form and not args.calib_copy and (bufs.fuse_permute or bufs.pre is None):
        del graph
        torch.cuda.empty_cache()
        tb = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, dt, save_pre=True, fuse_permute=False)
        tsteps = moe.forward_steps(x, wr, b, w13, w2, cfg.K, cfg.score, cfg.renorm, tb)

        def run_train():
            for _, call in tsteps:
                call()
        for _ in range(args.warmup):
            run_train()
        tgraph = capture(torch, run_train)
        tms = time_replays(torch, tgraph, args.warmup, args.steps)
        tkms, _ = time_steps(torch, tsteps, stream, args.steps)
        train = {"ms_per_step": tms, "tokens_per_s": cfg.T / (tms * 1e-3),
                 "gate_up_tflops": flops_up / (tkms["gemm_gate_up"] * 1e-3) / 1e12, "kernels_ms": tkms,
                 "form": "permute written, SwiGLU pre-activations saved (what a training step's forward does)"}
        del tgraph, tb, tsteps
        torch.cuda.empty_cache()
        graph = capture(torch, run_all)
    counts = bufs.counts.cpu().numpy()
    clock = None if args.no_clock or args.calib_copy else sample_clock(torch, graph.replay)
    # after the timed region; left out of the counter-calibration runs, whose own 512 MiB pass must
    # be the only elementwise kernel of its kind
    rates = stream_rates(torch) if not args.calib_copy else {"copy": float("nan"), "read": float("nan"),
                                                              "write": float("nan")}
    copy_gbs = rates["copy"]
    cpu = cpu_baseline(cfg, inp, args.cpu_seconds)
    if cpu is not None and cfg.name != "tiny_fp32":
        cpu["one_core"] = one_core_oracle(mi.CONFIGS["tiny_fp32"], cfg, inp)
    hbm_names = [n for n in ("router_route", "router", "permute", "combine") if n in kcold]
    hbm_cold = {n: nbytes[n] / (kcold[n]["median"] * 1e-3) / 1e9 for n in hbm_names}
    hbm_best = {n: nbytes[n] / (kcold[n]["min"] * 1e-3) / 1e9 for n in hbm_names}
    hbm_layer = {n: nbytes[n] / (kms[n] * 1e-3) / 1e9 for n in hbm_names if n in kms}
    sclk = clock.get("sclk_mhz_median") if clock else None

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
                         "down_tflops": tf_down, "flops_per_step": flops_up + flops_down,
                         "cold_median_tflops": {"gate_up": flops_up / (kcold["gemm_gate_up"]["median"] * 1e-3) / 1e12,
                                                "down": flops_down / (kcold["gemm_down"]["median"] * 1e-3) / 1e12}},
        "kernels_ms": kms,
        "kernels_cold_ms": kcold,
        "layer_replay_ms": layer_ms,
        "training_forward": train,
        "timing": {"value": "one HIP-graph replay of the layer per step",
                   "kernels_ms": "average of K eager passes of the layer, HIP events between the calls",
                   "layer_replay_ms": f"{args.cold_reps} graph replays each between its own HIP events, back to "
                                      "back (warm) and after a read-only 1 GiB pass (cold); median, min, mean",
                   "kernels_cold_ms": f"each kernel alone (and the standalone permute when the layer folds it "
                                      f"into the gate/up GEMM), {args.cold_reps} launches, a read-only 1 GiB pass "
                                      "before each (L2 and Infinity Cache cold)",
                   "eager_ms_per_step": eager_ms_per_step,
                   "eager_tokens_per_s": cfg.T / (eager_ms_per_step * 1e-3)},
        # HBM rates from the cold launches' median (min in hbm_gbs_best); in-layer rates may hit cache
        "hbm_gbs": hbm_cold,
        "hbm_gbs_best": hbm_best,
        "hbm_gbs_in_layer": hbm_layer,
        "hbm_frac": {k: {"of_spec": v / PEAK_HBM_GBS, "of_onbox_copy": v / copy_gbs} for k, v in hbm_cold.items()},
        "hbm_read_write_bytes": {k: list(nrw[k]) for k in hbm_cold},
        "onbox_copy_gbs": copy_gbs,
        "onbox_read_gbs": rates["read"],
        "onbox_write_gbs": rates["write"],
        "clock": clock,
        "load": {"min": int(counts.min()), "max": int(counts.max()), "empty": int((counts == 0).sum())},
        # the permute runs inside the gate/up GEMM's row loads (no permuted copy is written)
        "permute_folded_into_gate_up": bufs.fuse_permute,
        "roofline": {"kernel": "grouped GEMM gate/up + SwiGLU", "bound": "mfma", "achieved": tf_up,
                     "peak": peak, "unit": "TFLOP/s", "frac": tf_up / peak, "traffic": traffic,
                     **({"frac_of_peak_at_sustained_clock": tf_up / (peak * sclk / 2400.0)} if sclk else {})},
        "cpu_baseline": cpu,
        "input_generation_s": gen_s,
    }
    return out


def extra_lines(args, torch, moe, mi) -> dict:
    """Shorter runs of the other lines (at most 10 timed steps, 20 cold launches per kernel): the
    fine-grained and DeepSeek-V3-share forwards (no CPU sample, clock or training form), the
    backward and the MXFP8 forward, attached to the Mixtral-shaped forward line so that one default
    run measures them too. A failure is recorded in place of the line, never raised."""
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.cold_reps = min(args.steps, 10), min(args.warmup, 3), min(args.cold_reps, 20)
    sub.cpu_seconds, sub.no_clock, sub.no_train_form, sub.no_extras = 0.0, True, True, True
    fwd = ("grouped_gemm", "kernels_ms", "hbm_frac", "roofline")
    keep = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "dtype", "config", "timing")
    res = {}
    for name, fn, more in (("fine_grained", bench_forward, fwd), ("dsv3_share", bench_forward, fwd),
                           ("backward", bench_backward, ("gemm_tflops", "gemm_total_tflops", "kernels_ms")),
                           ("mxfp8", bench_mxfp8, ("grouped_gemm", "kernels_ms", "roofline"))):
        sub.workload = name if fn is bench_forward else "mixtral"
        try:
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            o = fn(sub, torch, moe, mi)
            res[name] = {k: o[k] for k in keep + more if k in o}
        except Exception as e:  # noqa: BLE001 - the headline line must still print
            res[name] = {"error": f"{type(e).__name__}: {e}"}
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def bench_backward(args, torch, moe, mi):
    """Backward of the Mixtral-shaped layer with one expert taking half of the slots and two none,
    the product's call sequence (layer_backward with the router): combine backward, SwiGLU-backward
    dgrad, down wgrad, gate/up dgrad, gate/up wgrad, permute backward, then the router's backward
    (d_gates -> d_logits -> dWr, and its share of dX); routing held fixed.  Timed as HIP-graph
    replays of the whole backward."""
    cfg = mi.CONFIGS["mixtral_bwd_skew"]
    torch.cuda.set_device(0)
    inp = mi.make(cfg)
    hot, dead = mi.skew_choice(cfg)
    dev = {k: to_dev(v, torch) for k, v in inp.items()}
    # the skewed routing is an input: the router product (the library's) with the dead experts
    # masked and the hot one lifted above every row's maximum
    raw = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(dev["x"], dev["w_router"], raw)
    torch.cuda.synchronize()
    logits = mi.skew_logits(raw.cpu().numpy(), hot, dead)
    dy = to_dev(mi.upstream_grad(cfg), torch)
    bufs = moe.MoEBuffers(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, torch.bfloat16, backward=True)
    logits_dev = to_dev(logits, torch)
    moe.layer_forward(dev["x"], dev["w_router"], None, dev["w13"], dev["w2"], cfg.K, cfg.score, cfg.renorm,
                      bufs, logits=logits_dev)
    stream = torch.cuda.current_stream()
    router = dict(logits=logits_dev, x=dev["x"], w_router=dev["w_router"], bias=None, score=cfg.score,
                  renorm=cfg.renorm)
    steps = moe.backward_steps(dy, dev["w13"], dev["w2"], cfg.K, bufs, router=router)

    def run_all():
        for _, call in steps:
            call()

    for _ in range(args.warmup):
        run_all()
    torch.cuda.synchronize()
    graph = capture(torch, run_all)
    ms = time_replays(torch, graph, args.warmup, args.steps)
    kms, eager_ms = time_steps(torch, steps, stream, args.steps)
    cold = ColdTimer(torch, stream)
    by_name = dict(steps)
    kcold = {n: cold.time(by_name[n], args.cold_reps) for n in ("combine_bwd", "permute_bwd", "route_bwd",
                                                                "router_bwd")}
    M = cfg.T * cfg.K
    fl = {"dgrad_down_dswiglu": 2.0 * M * cfg.d * cfg.F, "wgrad_down": 2.0 * M * cfg.d * cfg.F,
          "dgrad_gate_up": 2.0 * M * 2 * cfg.F * cfg.d, "wgrad_gate_up": 2.0 * M * 2 * cfg.F * cfg.d}
    tf = {k: fl[k] / (kms[k] * 1e-3) / 1e12 for k in fl}
    total_fl = sum(fl.values())
    # combine backward: dY read, dY_perm written, Y_perm read for the gate dot, gates and positions
    # read, d_gates written; permute backward: dX_perm read, dX written, positions read
    nb = {"combine_bwd": (cfg.T + 2 * M) * cfg.d * 2 + 12 * M, "permute_bwd": (M + cfg.T) * cfg.d * 2 + 4 * M,
          # d_logits pass: logits read, d_logits written, indices and d_gates read
          "route_bwd": 8.0 * cfg.T * cfg.E + 8 * M,
          # the router products: x read for dWr, dX read and written for its share
          "router_bwd": 3.0 * cfg.T * cfg.d * 2}
    out = {"metric": "MoE layer backward tokens/s (routing held fixed)", "value": cfg.T / (ms * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.K,
                      "ffn": cfg.F, "hot_expert_slots": int(bufs.counts.max().item()),
                      "empty_experts": int((bufs.counts == 0).sum().item())},
           "timing": {"value": "one HIP-graph replay of layer_backward (router included) per step",
                      "eager_ms_per_step": eager_ms},
           "gemm_tflops": tf, "gemm_frac_of_peak": {k: v / PEAK_BF16_TFLOPS for k, v in tf.items()},
           "gemm_total_tflops": total_fl / (sum(kms[k] for k in fl) * 1e-3) / 1e12,
           "kernels_ms": kms, "kernels_cold_ms": kcold,
           "hbm_gbs": {k: nb[k] / (kcold[k]["median"] * 1e-3) / 1e9 for k in kcold},
           "hbm_gbs_in_layer": {k: nb[k] / (kms[k] * 1e-3) / 1e9 for k in kcold}}
    return out


def bench_gemm_zipf(args, torch, moe, mi):
    """The two grouped GEMMs alone on 32768 rows in 32 groups of exact Zipf(1.2) sizes (ranks
    1..28 get floor(M r^-1.2 / H) rows, 4 groups none) at the DeepSeek-V3-share widths: the
    reading of "32768 routed tokens" as pre-routed rows with exact Zipf group sizes."""
    cfg = mi.CONFIGS["dsv3_share"]
    torch.cuda.set_device(0)
    M = 32768
    sizes = mi.zipf_group_sizes(M, cfg.E)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    a = mi.normal(cfg.seed, mi.TAG_X, (M, cfg.d), 1.0, True)
    wts = mi.make(cfg, rows=1)
    A, w13, w2 = to_dev(a, torch), to_dev(wts["w13"], torch), to_dev(wts["w2"], torch)
    offs = torch.from_numpy(off).cuda()
    H = torch.empty((M, cfg.F), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((M, cfg.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros((moe.moe_grouped_gemm_workspace_size(),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    steps = [("gemm_gate_up", lambda: moe.moe_grouped_gemm(A, w13, moe.MOE_LAYOUT_NK, offs, H, moe.MOE_EPI_SWIGLU,
                                                           workspace=ws)),
             ("gemm_down", lambda: moe.moe_grouped_gemm(H, w2, moe.MOE_LAYOUT_NK, offs, Y, moe.MOE_EPI_NONE,
                                                        workspace=ws))]

    def run_all():
        for _, call in steps:
            call()

    for _ in range(args.warmup):
        run_all()
    graph = capture(torch, run_all)
    ms = time_replays(torch, graph, args.warmup, max(args.steps, 100))
    kms, _ = time_steps(torch, steps, stream, max(args.steps, 100))
    fl_up, fl_down = 2.0 * M * 2 * cfg.F * cfg.d, 2.0 * M * cfg.F * cfg.d
    tf_up = fl_up / (kms["gemm_gate_up"] * 1e-3) / 1e12
    tf_down = fl_down / (kms["gemm_down"] * 1e-3) / 1e12
    out = {"metric": "grouped GEMM TFLOP/s, exact Zipf(1.2) group sizes (GEMMs only)",
           "value": (fl_up + fl_down) / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": max(args.steps, 100), "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "dsv3_share_zipf_rows", "rows": M, "groups": cfg.E, "d_model": cfg.d,
                      "ffn": cfg.F, "group_sizes": sorted(sizes.tolist(), reverse=True)},
           "kernels_ms": kms, "gate_up_tflops": tf_up, "down_tflops": tf_down,
           "frac_of_peak": {"gate_up": tf_up / PEAK_BF16_TFLOPS, "down": tf_down / PEAK_BF16_TFLOPS,
                            "both": (fl_up + fl_down) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}
    print(json.dumps(out), flush=True)


def bench_mxfp8(args, torch, moe, mi):
    """The bf16 layer forward with both expert GEMMs on MXFP8 operands: the tokens (then their
    codes are permuted) and H are quantised (32-value blocks, E8M0 scales, E4M3 values) inside
    every step, H by the gate/up GEMM's epilogue; the weights once, before the timed region, as
    stored MX weights would be."""
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
    # the gate/up GEMM writes H as MXFP8 (codes and scales) from its SwiGLU epilogue
    names = ["router_route", "quantize_x", "permute", "gemm_gate_up", "gemm_down", "combine"]

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
        moe.moe_grouped_gemm_mx(xq, xs, w13c, w13s, bufs.offsets, hq, moe.MOE_EPI_SWIGLU_MX, C_scales=hs,
                                workspace=bufs.gemm_ws)
        mark(4)
        moe.moe_grouped_gemm_mx(hq, hs, w2c, w2s, bufs.offsets, bufs.y_perm, moe.MOE_EPI_NONE, workspace=bufs.gemm_ws)
        mark(5)
        moe.moe_unpermute_combine(bufs.y_perm, bufs.slot_pos, bufs.gates, T, K, bufs.y)
        mark(6)

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
           "quantize_gbs": {"x": (T * d * 3 + T * d // 32) / (kms["quantize_x"] * 1e-3) / 1e9},
           "roofline": {"kernel": "MXFP8 grouped GEMM gate/up + SwiGLU", "bound": "mfma", "achieved": tf_up,
                        "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": tf_up / PEAK_FP8_TFLOPS,
                        "traffic": measured_traffic(args.traffic, f"{cfg.name}_mx/gemm_gate_up")},
           "cpu_baseline": None}
    return out


if __name__ == "__main__":
    main()
