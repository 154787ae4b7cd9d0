"""Plain, slow CPU oracle of the dropless MoE layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests, the package smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library: its only input
dependency is the seeded input generator (``moe_inputs``), which holds none of
the layer's arithmetic.

Source.  The page "Accelerating dropless MoE training in JAX with NVIDIA
Transformer Engine" (cited below as *TE-MoE*) describes the layer: a learned
router picks the Top-K experts of each token (introduction); every token is
processed by each expert it chose, with nothing dropped or padded (section
"How is dropless MoE different from capacity-based MoE?"); tokens are
dispatched into per-expert groups of variable length, the grouped MLP runs two
grouped GEMMs over those groups, and combine restores the original token order
(Figure 3 paragraph of "What specialised optimisations does dropless MoE
need?"); one grouped GEMM handles every expert at its real token count
("Optimisation 1: Grouped GEMM").  The page prints no formula.  Where it is
silent this oracle takes the plainest reading the rest supports:

* router logits are x . Wr^T (Wr stored [E, d]); keys are fp32(logit + bias),
  or the logits themselves when there is no bias;
* the K experts with the largest keys are chosen (ties: lower expert index;
  keys compared in the total order of fp32 bit patterns, so -0.0 < +0.0),
  listed by descending key;
* scores are a softmax over all E keys (or a sigmoid per key) and the K chosen
  scores are divided by their sum (renormalised gates);
* rows of each expert group are in ascending token order (a stable counting
  sort of the slots s = t*K + k);
* an expert is SwiGLU: h = silu(x Wg^T) * (x Wu^T), y = h W2^T, no biases;
  the first grouped GEMM is gate and up together (W13 = [Wg; Wu], [2F, d]),
  the second is the down projection (W2 [d, F]);
* the gates are applied in combine: y_t = sum_k g_tk * Y_perm[pos(t, k)];
* backward holds the routing fixed and yields dX, dW13, dW2 and d_gates;
  the router backward holds the top-K choice fixed and takes d_gates back
  through the scores to d_logits, then to dWr and the router's share of dx.

Arithmetic is fp64 from the exact input values with no intermediate rounding;
the only fp32 step is the key add, because it decides the integer routing and
both sides must take that decision in the same precision.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


# ----------------------------------------------------------------------------
# value decoding (bf16 inputs arrive as uint16 bit patterns)

def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of an fp32 / fp64 array or of bf16 bit patterns (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _fp32_order(v: np.float32) -> int:
    """Rank of an fp32 value in the total order of bit patterns (NaN excluded)."""
    u = int(np.float32(v).view(np.uint32))
    return (~u) & 0xFFFFFFFF if u & 0x80000000 else u | 0x80000000


# ----------------------------------------------------------------------------
# S0: router logits  (TE-MoE introduction: a learned router scores the experts)

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_j x[t, j] * Wr[e, j], computed in fp64, rounded once to fp32."""
    return (to_f64(x) @ to_f64(w_router).T).astype(np.float32)


# ----------------------------------------------------------------------------
# S1-S3: routing  (TE-MoE introduction: Top-K experts per token; "What are the
# challenges in MoE training?": every expert gets a different, data-dependent
# number of tokens, i.e. ragged groups)

@dataclass
class Routing:
    keys: np.ndarray      # [T, E] fp32  logit + bias
    idx: np.ndarray       # [T, K] int32 chosen experts, by descending key
    gates: np.ndarray     # [T, K] fp64  renormalised gate values
    counts: np.ndarray    # [E]    int64 slots per expert
    offsets: np.ndarray   # [E+1]  int64 exclusive prefix sum of counts
    slot_pos: np.ndarray  # [T*K]  int64 row of slot s in expert-contiguous order
    row_src: np.ndarray   # [T*K]  int64 slot held by permuted row r (inverse of slot_pos)


def scores(k64: np.ndarray, score: int) -> np.ndarray:
    """S1b: scores of one token's keys in fp64: a softmax over all E keys, or a sigmoid per key."""
    if score == SCORE_SOFTMAX:
        z = np.exp(k64 - k64.max())
        return z / z.sum()
    if score == SCORE_SIGMOID:
        return 1.0 / (1.0 + np.exp(-k64))
    raise ValueError("score must be softmax (0) or sigmoid (1)")


def gates_from_keys(k64: np.ndarray, chosen, score: int, renorm: bool) -> np.ndarray:
    """S1b-S1c: the chosen experts' scores, divided by their sum when renormalising."""
    sel = scores(k64, score)[list(chosen)]
    return sel / sel.sum() if renorm else sel


def route(logits: np.ndarray, bias: np.ndarray | None, K: int, score: int = SCORE_SOFTMAX,
          renorm: bool = True) -> Routing:
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    if bias is None:
        keys = logits.copy()              # no add: a -0.0 logit stays -0.0
    else:
        keys = logits + np.asarray(bias, np.float32)[None, :]   # fp32 add, nearest even

    idx = np.zeros((T, K), np.int32)
    gates = np.zeros((T, K), np.float64)
    for t in range(T):
        row = keys[t]
        # S1a: order experts by (key descending, expert ascending); keep the first K
        order = sorted(range(E), key=lambda e: (-_fp32_order(row[e]), e))
        chosen = order[:K]
        idx[t] = chosen
        gates[t] = gates_from_keys(row.astype(np.float64), chosen, score, renorm)

    # S2: per-expert histogram and its exclusive prefix sum
    M = T * K
    counts = np.zeros(E, np.int64)
    for s_ in range(M):
        counts[idx.flat[s_]] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    # S3: stable counting sort of the slots by expert
    cursor = offsets[:E].copy()
    slot_pos = np.zeros(M, np.int64)
    row_src = np.zeros(M, np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            s_ = t * K + k
            slot_pos[s_] = cursor[e]
            row_src[cursor[e]] = s_
            cursor[e] += 1
    return Routing(keys, idx, gates, counts, offsets, slot_pos, row_src)


# ----------------------------------------------------------------------------
# S4: permute / dispatch into expert-contiguous order (TE-MoE Figure 3 paragraph)

def permute(x: np.ndarray, row_src: np.ndarray, K: int) -> np.ndarray:
    """X_perm[r] = x[row_src[r] // K]: a copy of the token's row, bits unchanged."""
    x = np.asarray(x)
    out = np.empty((len(row_src),) + x.shape[1:], dtype=x.dtype)
    for r, s_ in enumerate(row_src):
        out[r] = x[s_ // K]
    return out


# ----------------------------------------------------------------------------
# S5, S6: the two grouped GEMMs ("Optimisation 1: Grouped GEMM": every expert
# matmul at its actual token count; here a plain loop over experts)

def grouped_gemm(a: np.ndarray, b: np.ndarray, offsets: np.ndarray, b_layout: str = "nk") -> np.ndarray:
    """C[rows of group g] = A[rows of g] . B_g^T  (b_layout "nk": B [G, N, Kd])
    or A[rows of g] . B_g  (b_layout "kn": B [G, Kd, N]); fp64.  Weights are
    widened to fp64 one group at a time, and only for groups that own rows."""
    A = to_f64(a)
    G = b.shape[0]
    N = b.shape[1] if b_layout == "nk" else b.shape[2]
    C = np.zeros((A.shape[0], N), np.float64)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        Bg = to_f64(b[g])
        C[lo:hi] = A[lo:hi] @ (Bg.T if b_layout == "nk" else Bg)
    return C


def silu(v: np.ndarray) -> np.ndarray:
    # below v = -709, exp(-v) overflows to inf and v / inf is the limit, 0: the overflow is expected
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu(pre: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up, with pre = [gate | up] along the last axis."""
    F = pre.shape[-1] // 2
    return silu(pre[..., :F]) * pre[..., F:]


def grouped_wgrad(x: np.ndarray, dy: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """dW[g] = dY_g^T . X_g over the rows of group g, [G, N, Kd]; zeros for empty groups."""
    X = to_f64(x)
    D = to_f64(dy)
    G = len(offsets) - 1
    dW = np.zeros((G, D.shape[1], X.shape[1]), np.float64)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            dW[g] = D[lo:hi].T @ X[lo:hi]
    return dW


# ----------------------------------------------------------------------------
# S7: unpermute + gate-weighted combine (TE-MoE Figure 3 paragraph: combine
# restores the original token order)

def combine(y_perm: np.ndarray, slot_pos: np.ndarray, gates: np.ndarray | None, T: int, K: int) -> np.ndarray:
    """Y[t] = sum_{k<K} g_tk * Y_perm[slot_pos[t*K+k]]  (g = 1 when gates is None)."""
    Yp = to_f64(y_perm)
    Y = np.zeros((T, Yp.shape[1]), np.float64)
    for t in range(T):
        for k in range(K):
            g = 1.0 if gates is None else float(gates[t, k])
            Y[t] += g * Yp[slot_pos[t * K + k]]
    return Y


def combine_backward(dy, y_perm, slot_pos, gates, T: int, K: int):
    """Adjoint of the gate-weighted combine:
    dY_perm[slot_pos[s]] = g_s dY[t] and d_gate_s = <dY[t], Y_perm[slot_pos[s]]>."""
    dY = to_f64(dy)
    Yp = to_f64(y_perm)
    dy_perm = np.zeros((T * K, dY.shape[1]), np.float64)
    d_gates = np.zeros((T, K), np.float64)
    for t in range(T):
        for k in range(K):
            p = slot_pos[t * K + k]
            dy_perm[p] = float(gates[t, k]) * dY[t]
            d_gates[t, k] = float(dY[t] @ Yp[p])
    return dy_perm, d_gates


def swiglu_backward(dh, pre):
    """d[gate | up] of h = silu(gate) * up:  dG = dH U silu'(G), dU = dH silu(G),
    with silu'(G) = s (1 + G (1 - s)), s = sigmoid(G)."""
    dH = to_f64(dh)
    P = to_f64(pre)
    F = P.shape[1] // 2
    G, U = P[:, :F], P[:, F:]
    sg = 1.0 / (1.0 + np.exp(-G))
    return np.concatenate([dH * U * sg * (1.0 + G * (1.0 - sg)), dH * G * sg], axis=1)


# ----------------------------------------------------------------------------
# the whole forward layer

def forward(x, w_router, bias, w13, w2, K, score=SCORE_SOFTMAX, renorm=True, logits=None) -> dict:
    """Router -> dispatch -> two grouped GEMMs -> combine.  Returns every intermediate.

    ``logits`` (fp32 [T, E]) replaces the router product when given."""
    T = np.asarray(x).shape[0]
    if logits is None:
        logits = router_logits(x, w_router)
    r = route(logits, bias, K, score, renorm)
    x_perm = permute(x, r.row_src, K)
    pre = grouped_gemm(x_perm, w13, r.offsets, "nk")          # [M, 2F]
    h = swiglu(pre)                                           # [M, F]
    y_perm = grouped_gemm(h, w2, r.offsets, "nk")             # [M, d]
    y = combine(y_perm, r.slot_pos, r.gates, T, K)
    return {"logits": logits, "routing": r, "x_perm": x_perm, "pre": pre, "h": h,
            "y_perm": y_perm, "y": y}


def backward(dy, fwd: dict, w13, w2, K) -> dict:
    """Gradients of <dY, Y> with the routing held fixed.

    B1 combine backward: dY_perm[pos(s)] = g_s dY[t], d_gate_s = <dY[t], Y_perm[pos(s)]>
    B2 down dgrad + SwiGLU backward: dH = dY_perm_e W2_e, dA = [dG | dU]
    B3 down wgrad:  dW2_e = dY_perm_e^T H_e
    B4 gate/up dgrad: dX_perm_e = dA_e W13_e
    B5 gate/up wgrad: dW13_e = dA_e^T X_perm_e
    B6 permute backward: dX[t] = sum_k dX_perm[pos(t, k)]
    """
    r: Routing = fwd["routing"]
    T = np.asarray(dy).shape[0]
    dy_perm, d_gates = combine_backward(dy, fwd["y_perm"], r.slot_pos, r.gates, T, K)
    pre = fwd["pre"]
    dh = grouped_gemm(dy_perm, w2, r.offsets, "kn")           # [M, F]
    d_pre = swiglu_backward(dh, pre)
    dw2 = grouped_wgrad(fwd["h"], dy_perm, r.offsets)        # [E, d, F]
    dx_perm = grouped_gemm(d_pre, w13, r.offsets, "kn")       # [M, d]
    dw13 = grouped_wgrad(fwd["x_perm"], d_pre, r.offsets)    # [E, 2F, d]
    dx = combine(dx_perm, r.slot_pos, None, T, K)
    return {"dy_perm": dy_perm, "d_gates": d_gates, "dh": dh, "d_pre": d_pre, "dw2": dw2,
            "dx_perm": dx_perm, "dw13": dw13, "dx": dx}


# ----------------------------------------------------------------------------
# Single rows and single weight-gradient entries of the same layer.  A row of
# the expert-contiguous order depends only on its own token, its expert and
# that expert's weights, and an entry dW_e[n, k] only on column n of one factor
# and column k of the other over the group's rows; these functions evaluate
# exactly the definitions of forward() and backward() for the rows and entries
# asked for, so that layers too large to form whole can still be checked.

def group_of_rows(routing: Routing, rows) -> np.ndarray:
    """Expert owning each expert-contiguous row: offsets[e] <= r < offsets[e + 1]."""
    rows = np.asarray(rows, np.int64)
    return np.searchsorted(routing.offsets, rows, side="right") - 1


def layer_rows(x, w13, w2, routing: Routing, rows, K: int) -> dict:
    """x_perm, pre, h and y_perm of the expert-contiguous rows ``rows`` (S4-S6)."""
    rows = np.asarray(rows, np.int64)
    x = np.asarray(x)
    tok = routing.row_src[rows] // K
    grp = group_of_rows(routing, rows)
    F = w13.shape[1] // 2
    out = {"x_perm": x[tok], "pre": np.zeros((len(rows), 2 * F)), "h": np.zeros((len(rows), F)),
           "y_perm": np.zeros((len(rows), w2.shape[1]))}
    for e in np.unique(grp):
        sel = np.nonzero(grp == e)[0]
        pre = to_f64(x[tok[sel]]) @ to_f64(w13[e]).T
        h = swiglu(pre)
        out["pre"][sel] = pre
        out["h"][sel] = h
        out["y_perm"][sel] = h @ to_f64(w2[e]).T
    return out


def backward_rows(x, dy, w13, w2, routing: Routing, rows, K: int) -> dict:
    """dy_perm, d_pre and dx_perm of the expert-contiguous rows ``rows`` (B1, B2, B4)."""
    rows = np.asarray(rows, np.int64)
    slot = routing.row_src[rows]
    tok, kk = slot // K, slot % K
    grp = group_of_rows(routing, rows)
    fw = layer_rows(x, w13, w2, routing, rows, K)
    dy_perm = routing.gates[tok, kk][:, None] * to_f64(np.asarray(dy)[tok])
    d_pre = np.zeros_like(fw["pre"])
    dx_perm = np.zeros((len(rows), w13.shape[2]))
    for e in np.unique(grp):
        sel = np.nonzero(grp == e)[0]
        dh = dy_perm[sel] @ to_f64(w2[e])
        d_pre[sel] = swiglu_backward(dh, fw["pre"][sel])
        dx_perm[sel] = d_pre[sel] @ to_f64(w13[e])
    return {"dy_perm": dy_perm, "d_pre": d_pre, "dx_perm": dx_perm}


def wgrad_entries(x, dy, w13, w2, routing: Routing, K: int, e: int, which: str, n_idx, k_idx) -> np.ndarray:
    """Entries [n_idx][:, k_idx] of one expert's weight gradient (B3 / B5):
    which = "w2":  dW2_e[n, k]  = sum over the group's rows r of dy_perm[r, n] * h[r, k];
    which = "w13": dW13_e[n, k] = sum over the group's rows r of d_pre[r, n] * x_perm[r, k].
    Only the columns of h or d_pre that the entries need are formed."""
    n_idx = np.asarray(n_idx, np.int64)
    k_idx = np.asarray(k_idx, np.int64)
    lo, hi = int(routing.offsets[e]), int(routing.offsets[e + 1])
    F = w13.shape[1] // 2
    if hi == lo:
        return np.zeros((len(n_idx), len(k_idx)))
    slot = routing.row_src[lo:hi]
    tok, kk = slot // K, slot % K
    X = to_f64(np.asarray(x)[tok])                                       # x_perm rows of the group
    dYp = routing.gates[tok, kk][:, None] * to_f64(np.asarray(dy)[tok])  # dy_perm rows of the group
    W13 = w13[e]

    def pre_cols(j):   # [gate | up] pre-activations of the group at hidden columns j
        return np.concatenate([X @ to_f64(W13[j]).T, X @ to_f64(W13[F + j]).T], axis=1)

    if which == "w2":
        h = swiglu(pre_cols(k_idx))                                     # h[:, k_idx]
        return dYp[:, n_idx].T @ h
    if which == "w13":
        j = n_idx % F
        dh = dYp @ to_f64(w2[e][:, j])                                  # dh[:, j]
        dpre = swiglu_backward(dh, pre_cols(j))                         # [dG | dU] at columns j
        m = len(j)
        cols = np.where(n_idx < F, np.arange(m), m + np.arange(m))
        return dpre[:, cols].T @ X[:, k_idx]
    raise ValueError("which must be 'w2' or 'w13'")


# ----------------------------------------------------------------------------
# Router backward.  The router is learned (TE-MoE introduction), so training
# needs the gradient of the loss with respect to its weights and inputs.  The
# top-K choice is a discrete decision and is held fixed; the gradient flows
# through the scores and their renormalisation (S1b-S1c), then through the
# router product (S0).  A bias is a constant offset of the keys: d key = d logit.

def route_backward(keys: np.ndarray, idx: np.ndarray, d_gates: np.ndarray, score: int = SCORE_SOFTMAX,
                   renorm: bool = True) -> np.ndarray:
    """d_logits[t, e] = sum_k d_gates[t, k] * d gate[t, k] / d key[t, e], fp64 [T, E].

    The chain rule step by step for each token: first back through the
    renormalisation g_k = s_k / S (S = sum of the chosen scores), giving d s for
    the chosen experts (0 for the rest), then back through the score function:
    the softmax Jacobian ds/dkey = diag(s) - s s^T, or s (1 - s) for a sigmoid."""
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    K = idx.shape[1]
    d_gates = np.asarray(d_gates, np.float64).reshape(T, K)
    out = np.zeros((T, E), np.float64)
    for t in range(T):
        chosen = [int(e) for e in idx[t]]
        s = scores(keys[t], score)
        dg = d_gates[t]
        ds = np.zeros(E, np.float64)
        if renorm:
            S = s[chosen].sum()
            g = s[chosen] / S
            # d g_k / d s_j = (delta_kj - g_k) / S over the chosen j
            for j in range(K):
                ds[chosen[j]] += sum(dg[k] * ((1.0 if k == j else 0.0) - g[k]) / S for k in range(K))
        else:
            for k in range(K):
                ds[chosen[k]] += dg[k]
        if score == SCORE_SOFTMAX:
            out[t] = s * ds - s * np.dot(s, ds)
        else:
            out[t] = ds * s * (1.0 - s)
    return out


def router_backward(d_logits: np.ndarray, x: np.ndarray, w_router: np.ndarray):
    """Backward of logits = x . Wr^T: dWr = d_logits^T . x  [E, d], dx = d_logits . Wr  [T, d]; fp64."""
    dl = np.asarray(d_logits, np.float64)
    return dl.T @ to_f64(x), dl @ to_f64(w_router)


# ----------------------------------------------------------------------------
# MXFP8 block scaling of the expert matmuls (TE-MoE "Optimisation 1": on newer
# GPUs the grouped GEMM path takes MXFP8 operands from grouped quantisation).
# The pages name the format only.  Its definition is the OCP Microscaling (MX)
# format: every 32 consecutive elements along the reduction axis share one
# power-of-two scale stored as E8M0 (code c means 2^(c - 127)); the elements
# are FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
# finite value 448, smallest subnormal 2^-9, no infinities).  The conversion
# reads: shared exponent = floor(log2(max |v|)) - 8 (8 is E4M3's largest
# exponent), clamped to [-127, 127]; a block of zeros takes code 0; each
# element is v / 2^shared rounded to nearest even and saturated to +-448.

MX_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an FP8 E4M3 code (0x7F / 0xFF are NaN)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code (ties to even mantissa), saturating to +-448; v finite."""
    v = float(v)
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < 2.0 ** -6:                       # subnormal grid of 2^-9
        q = round(a * 2.0 ** 9)             # Python's round: ties to even
        return sign | q                     # q == 8 is the smallest normal, code 0x08
    f, e = math.frexp(a)                    # a = f 2^e, f in [0.5, 1)
    e -= 1                                  # a = (2 f) 2^e, 2 f in [1, 2)
    m = round((2.0 * f - 1.0) * 8.0)
    if m == 8:
        e, m = e + 1, 0
    return sign | ((e + 7) << 3) | m


def mx_quantize(a: np.ndarray):
    """MXFP8 of a [R, K] array (K a multiple of 32) along its last axis.

    Returns (codes uint8 [R, K], scales uint8 [R, K / 32]) with value = e4m3(code) * 2^(scale - 127)."""
    v = to_f64(a)
    R, K = v.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((R, K), np.uint8)
    scales = np.zeros((R, K // MX_BLOCK), np.uint8)
    for r in range(R):
        for b in range(K // MX_BLOCK):
            blk = v[r, b * MX_BLOCK:(b + 1) * MX_BLOCK]
            amax = float(np.max(np.abs(blk)))
            if amax == 0.0:
                shared = -127
            else:
                shared = min(127, max(-127, math.frexp(amax)[1] - 1 - 8))
            scales[r, b] = shared + 127
            for i, x in enumerate(blk):
                codes[r, b * MX_BLOCK + i] = e4m3_encode(math.ldexp(float(x), -shared))
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 values of MXFP8 codes and their block scales."""
    table = np.array([e4m3_decode(c) for c in range(256)], np.float64)
    val = table[codes]
    factor = np.exp2(scales.astype(np.float64) - 127.0)
    return val * np.repeat(factor, MX_BLOCK, axis=-1)


def grouped_gemm_mx(a_codes, a_scales, b_codes, b_scales, offsets: np.ndarray) -> np.ndarray:
    """The grouped GEMM (N-by-K weights) on the values the MXFP8 operands represent, in fp64."""
    a = mx_dequantize(a_codes, a_scales)
    G, N, K = b_codes.shape
    b = mx_dequantize(b_codes.reshape(G * N, K), b_scales.reshape(G * N, K // MX_BLOCK)).reshape(G, N, K)
    return grouped_gemm(a, b, offsets, "nk")


# ----------------------------------------------------------------------------
# independent evaluations used to pin the per-expert loop

def dense_gate_matrix(routing: Routing, E: int) -> np.ndarray:
    """G[t, e] = gate of expert e for token t, 0 where e was not chosen."""
    T, K = routing.idx.shape
    Gm = np.zeros((T, E), np.float64)
    for t in range(T):
        for k in range(K):
            Gm[t, routing.idx[t, k]] = routing.gates[t, k]
    return Gm


def dense_layer(x, gate_matrix: np.ndarray, w13, w2) -> np.ndarray:
    """Every expert on every token, masked by the dense gate matrix:
    Y = sum_e G[:, e] * (silu(X Wg_e^T) * (X Wu_e^T)) W2_e^T.
    (Experts whose gate column is all zero add nothing and are skipped.)"""
    X = to_f64(x)
    E = w13.shape[0]
    Y = np.zeros((X.shape[0], w2.shape[1]), np.float64)
    for e in range(E):
        if not np.any(gate_matrix[:, e]):
            continue
        Y += gate_matrix[:, e:e + 1] * (swiglu(X @ to_f64(w13[e]).T) @ to_f64(w2[e]).T)
    return Y


def capacity_layer(x, routing: Routing, w13, w2, capacity: int) -> np.ndarray:
    """Capacity-based contrast (TE-MoE "How is dropless MoE different from
    capacity-based MoE?"): each expert takes at most ``capacity`` slots in
    token order and the rest are dropped (contribute zero)."""
    T, K = routing.idx.shape
    E = w13.shape[0]
    taken = np.zeros(E, np.int64)
    Gm = np.zeros((T, E), np.float64)
    for t in range(T):
        for k in range(K):
            e = routing.idx[t, k]
            if taken[e] < capacity:
                Gm[t, e] += routing.gates[t, k]
                taken[e] += 1
    return dense_layer(x, Gm, w13, w2)
