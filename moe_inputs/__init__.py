"""Seeded synthetic inputs for the dropless MoE layer.

This module is the only code that the CPU oracle and the GPU path share.  It
draws random tensors and encodes them; it holds none of the layer's own
arithmetic (no router product, no scores, no routing, no expert math).

Workloads follow the shapes the on-subject page ("Accelerating dropless MoE
training in JAX with NVIDIA Transformer Engine") motivates: Mixtral-, Qwen- and
DeepSeek-style MoE layers (its introduction), learned routers whose load is
skewed and differs from batch to batch ("What are the challenges in MoE
training?"), and experts that receive no tokens at all.  The pages print no
shapes; the sizes below are the five workloads this library is measured on.

Random streams
--------------
Every tensor has an integer tag.  Its flat element range is cut into chunks
of ``CHUNK`` elements, and chunk ``c`` is drawn from
``PCG64(SeedSequence([seed, tag, c])).standard_normal(float32)`` and scaled by
the tensor's standard deviation in fp32.  Chunks are independent, so they are
drawn on a thread pool, and any prefix of rows is reproducible on its own.
bf16 tensors are the fp32 draws rounded to nearest-even and are handed out as
``uint16`` bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1 << 22

# tensor tags of the random streams
TAG_X, TAG_WR, TAG_W13, TAG_W2, TAG_BIAS, TAG_RANKS, TAG_DY, TAG_SKEW = 1, 2, 3, 4, 5, 6, 7, 8

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_chunk(seed: int, tag: int, c: int, n: int, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, c])))
    a = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def normal(seed: int, tag: int, shape, std: float, bf16: bool, rows: int | None = None) -> np.ndarray:
    """N(0, std^2) tensor of ``shape`` from stream (seed, tag).

    With ``rows`` set, only the first ``rows`` rows of the full tensor are
    produced (bitwise equal to the same rows of the full draw).
    """
    shape = tuple(int(s) for s in shape)
    if rows is not None:
        shape = (int(rows),) + shape[1:]
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def job(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        a = _draw_chunk(seed, tag, c, CHUNK, std)[: hi - lo]
        out[lo:hi] = f32_to_bf16_bits(a) if bf16 else a

    if nchunks <= 1:
        for c in range(nchunks):
            job(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(nchunks)))
    return out.reshape(shape)


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload: layer shapes, dtypes, router recipe and seed."""
    name: str
    seed: int
    T: int          # tokens
    d: int          # model width
    E: int          # experts
    K: int          # experts per token
    F: int          # expert FFN width (SwiGLU hidden size)
    bf16: bool      # bf16 inputs/outputs (fp32 accumulate); else all fp32
    score: int = SCORE_SOFTMAX
    renorm: bool = True
    x_std: float = 1.0
    wr_std: float | None = None     # router weight std; None = 1/sqrt(d)
    w_std: float | None = None      # expert weight std; None = 1/sqrt(d)
    bias: str = "none"              # "none" | "normal" | "zipf_ranks"
    skew: str = "none"              # "none" | "hot_dead" (logit override, backward workload)
    dy_seed: int | None = None      # seed of the upstream gradient dY (backward workloads)
    notes: str = field(default="", compare=False)

    @property
    def M(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "MoEConfig":
        return replace(self, T=int(T))


CONFIGS = {
    "tiny_fp32": MoEConfig(
        "tiny_fp32", seed=1, T=256, d=128, E=8, K=2, F=256, bf16=False,
        notes="tiny fp32 layer: x~N(0,1), all weights N(0,1/d), softmax top-2"),
    "mixtral": MoEConfig(
        "mixtral", seed=2, T=8192, d=4096, E=8, K=2, F=14336, bf16=True, wr_std=0.02,
        notes="Mixtral-shaped layer: near-uniform load"),
    "fine_grained": MoEConfig(
        "fine_grained", seed=3, T=16384, d=2048, E=128, K=8, F=768, bf16=True, wr_std=0.02,
        bias="normal", notes="many small experts; per-expert logit bias N(0,1) skews the load"),
    "dsv3_share": MoEConfig(
        "dsv3_share", seed=4, T=32768, d=7168, E=32, K=8, F=2048, bf16=True, wr_std=0.02,
        score=SCORE_SIGMOID, bias="zipf_ranks",
        notes="one GPU's share of a DeepSeek-V3-shaped layer: sigmoid scores, "
              "Zipf-like load by rank, 4 experts with no tokens"),
    "mixtral_bwd_skew": MoEConfig(
        "mixtral_bwd_skew", seed=2, T=8192, d=4096, E=8, K=2, F=14336, bf16=True, wr_std=0.02,
        skew="hot_dead", dy_seed=5,
        notes="backward of the Mixtral-shaped layer: one expert takes half of the slots, two take none"),
}


def router_bias(cfg: MoEConfig) -> np.ndarray | None:
    """Per-expert fp32 bias added to the router logits, or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return normal(cfg.seed, TAG_BIAS, (cfg.E,), 1.0, bf16=False)
    if cfg.bias == "zipf_ranks":
        # A Zipf-like load by rank: expert of rank r gets logit offset
        # -s * (sqrt(6)/pi) * sigma_l * ln r, which gives load ~ r^-s for
        # Gumbel-like logit noise of std sigma_l; the 4 last ranks get -inf,
        # so those experts receive no tokens.
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, TAG_RANKS])))
        ranks = g.permutation(cfg.E) + 1
        wr_std = cfg.wr_std if cfg.wr_std is not None else 1.0 / math.sqrt(cfg.d)
        sigma_l = wr_std * math.sqrt(cfg.d) * cfg.x_std
        s = 1.2
        live = cfg.E - 4
        b = np.where(ranks <= live,
                     -s * (math.sqrt(6.0) / math.pi) * sigma_l * np.log(ranks.astype(np.float64)),
                     -np.inf)
        return b.astype(np.float32)
    raise ValueError(cfg.bias)


def zipf_group_sizes(M: int, E: int, dead: int = 4, s: float = 1.2, seed: int = 4) -> np.ndarray:
    """Rows per expert group for a GEMM-only workload with an exact Zipf(s) load: the group of
    rank r (1 .. E - dead) gets floor(M r^-s / H) rows, H = sum of r^-s over those ranks, the
    remainder goes to rank 1, and the last ``dead`` ranks get none.  Ranks are dealt to
    experts by the DeepSeek-V3-share permutation stream (tag TAG_RANKS), so the largest
    group is not always the first."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAG_RANKS])))
    ranks = g.permutation(E) + 1
    live = E - dead
    w = np.arange(1, live + 1, dtype=np.float64) ** -s
    by_rank = np.floor(M * w / w.sum()).astype(np.int64)
    by_rank[0] += M - by_rank.sum()
    sizes = np.zeros(E, np.int64)
    for e in range(E):
        if ranks[e] <= live:
            sizes[e] = by_rank[ranks[e] - 1]
    return sizes


def make(cfg: MoEConfig, rows: int | None = None, weights: bool = True) -> dict:
    """All layer inputs of ``cfg`` as host arrays.

    x [T,d], w_router [E,d] (router weight, row e scores expert e),
    w13 [E,2F,d] (rows 0..F-1 gate, F..2F-1 up), w2 [E,d,F], bias [E] fp32 or None.
    bf16 tensors are uint16 bit patterns; fp32 tensors are float32.
    ``rows`` limits x to its first rows (the weights are the full ones).
    """
    T = cfg.T if rows is None else min(int(rows), cfg.T)
    wr_std = cfg.wr_std if cfg.wr_std is not None else 1.0 / math.sqrt(cfg.d)
    w_std = cfg.w_std if cfg.w_std is not None else 1.0 / math.sqrt(cfg.d)
    out = {
        "x": normal(cfg.seed, TAG_X, (cfg.T, cfg.d), cfg.x_std, cfg.bf16, rows=T),
        "w_router": normal(cfg.seed, TAG_WR, (cfg.E, cfg.d), wr_std, cfg.bf16),
        "bias": router_bias(cfg),
    }
    if weights:
        out["w13"] = normal(cfg.seed, TAG_W13, (cfg.E, 2 * cfg.F, cfg.d), w_std, cfg.bf16)
        out["w2"] = normal(cfg.seed, TAG_W2, (cfg.E, cfg.d, cfg.F), w_std, cfg.bf16)
    return out


def upstream_grad(cfg: MoEConfig, rows: int | None = None) -> np.ndarray:
    """dY [T,d] ~ N(0,1) for backward workloads."""
    seed = cfg.dy_seed if cfg.dy_seed is not None else cfg.seed + 1000
    return normal(seed, TAG_DY, (cfg.T, cfg.d), 1.0, cfg.bf16, rows=rows)


def skew_choice(cfg: MoEConfig) -> tuple[int, list[int]]:
    """(hot expert, dead experts) of the adversarial backward workload."""
    seed = cfg.dy_seed if cfg.dy_seed is not None else cfg.seed + 1000
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAG_SKEW])))
    pick = g.choice(cfg.E, 3, replace=False)
    return int(pick[0]), [int(pick[1]), int(pick[2])]


def skew_logits(logits: np.ndarray, hot: int, dead: list[int]) -> np.ndarray:
    """Adversarial load: dead experts' logits become -inf and the hot expert's
    logit becomes (row max + 1), so every token picks the hot expert (half of
    the slots at K=2) and never a dead one; gates stay O(1)."""
    out = np.array(logits, dtype=np.float32, copy=True)
    out[:, dead] = -np.inf
    out[:, hot] = out.max(axis=1) + np.float32(1.0)
    return out
