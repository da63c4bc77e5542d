"""CPU oracle: the forward pass of one mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the package and
the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP path and imports nothing from it.

Plain numpy.  Floating-point work is done in float64 on the stored input values
(bf16 inputs arrive widened to float32, which is exact) and rounded once, with
round-to-nearest-even, to the output type.  No blocking, fusion or reordering
beyond what the definitions below state; matrix products and sorts are numpy
library calls.

Sources (titles of the pages this follows):
  [TM]  Transformers & Math, module 17 "Mixture of Experts", sections 17.1-17.5
        and the exercises.
  [MIN] ML Interview Notes, "Mixture of Experts: Sparse FFNs, Routers, and Shared
        Experts": the Router and MoELayer listings, "Auxiliary load-balancing
        loss", "Capacity factor".
  [UD]  Understanding Data, "Mixture of experts" (AI engineering visualised),
        "The maths": gate, capacity, load imbalance.
  [RS]  The Residual Stream, "Mixture of Experts: More Parameters, Same FLOPs":
        "The router" (equation and worked example), "Keeping the load even",
        "An MoE tiny GPT" (the MoE listing), "Counting real models".
  [LT]  Latent, "Mixture of experts": "Where the experts live" (gate equation),
        "Keeping the load balanced" (balance equation).

Readings where the pages are silent or disagree (each also listed in the design
notes of the repository):
  * f_i is the share of token *assignments* (sum over experts = 1), as in the
    [RS] listing (counts / counts.sum()) and [LT]; the [MIN] listing's one-hot
    sum is k times this.  f_i and the max/mean load are taken on demand, before
    any capacity cut ([UD] "Load imbalance").
  * P_i is the mean of the softmax over all E experts in every score mode
    ([MIN] load_balancing_loss takes the full softmax although its router
    softmaxes only the chosen k).
  * Selection is on float32 keys: the router scores, sigmoid(scores) in the
    sigmoid mode, or, with a selection bias, softmax(s) + b / s + b /
    sigmoid(s) + b by mode (the [RS] listing adds the bias to the softmax
    probabilities).  Equal keys go to the lower expert index; slots are ordered
    by descending key.
  * In the sigmoid mode the weights are the chosen sigmoid scores normalized over
    the chosen k, always ([RS] "The router"); P_i stays the mean softmax.
  * An expert over capacity keeps the tokens that reach it first in ascending
    token order; a dropped slot contributes nothing and the token's other
    weights are not renormalized ([TM] 17.5; [MIN] "Capacity factor").
  * The shared expert is added unweighted ([TM] 17.2 equation; [MIN] MoELayer).
  * SiLU(z) = z / (1 + e^-z).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Optional

import numpy as np

SOFTMAX_THEN_TOPK = 0
TOPK_THEN_SOFTMAX = 1
SIGMOID_THEN_TOPK = 2
NEAR_TIE_GAP = 1e-4


# ----------------------------------------------------------------------------
# Rounding of float64 results to the stored output types.

def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), in one step.
    Returned as float32 holding the bf16 value exactly (finite, normal inputs)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)             # 8 significant bits, half to even
    return np.ldexp(r, e - 8).astype(np.float32)


def bf16_value_to_bits(v32: np.ndarray) -> np.ndarray:
    """Bit pattern of float32 values that are already exact bfloat16 values."""
    return (np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(v) if dtype == "bf16" else np.asarray(v, dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# Router.

def router_scores(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """One score per expert and token, s = W_r x ([LT] "Where the experts live";
    [RS] "The router": a single linear layer; [MIN] Router.gate, nn.Linear
    without bias).  W_r is held (E, d).  The optional per-expert bias is added
    to the score.  Exact products summed in float64, rounded once to float32."""
    s = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        s = s + np.asarray(bias, np.float64)[None, :]
    return s.astype(np.float32)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s_i) / sum_j exp(s_j), float64, with the row maximum subtracted first."""
    s = np.asarray(s, np.float64)
    z = np.exp(s - s.max(axis=axis, keepdims=True))
    return z / z.sum(axis=axis, keepdims=True)


def sigmoid(s: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-s)), float64."""
    return 1.0 / (1.0 + np.exp(-np.asarray(s, np.float64)))


def selection_keys(scores: np.ndarray, mode: int, select_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """What top-k ranks, per token and expert.

    Without a selection bias: the score itself (softmax and top-k-first modes;
    softmax is monotonic, so ranking the probabilities ranks the scores), or
    sigmoid(score) in the sigmoid mode.
    With a selection bias b ([RS] "Keeping the load even", bias balancing, and the
    MoE listing's balance="bias": the bias is added only to what chooses the
    top k, never to the weights): softmax(s) + b, s + b (top-k-first), or
    sigmoid(s) + b.  Returned as float32, the precision the selection runs in."""
    s = np.asarray(scores, np.float64)
    if select_bias is None:
        key = sigmoid(s) if mode == SIGMOID_THEN_TOPK else s
    else:
        b = np.asarray(select_bias, np.float64)[None, :]
        if mode == SOFTMAX_THEN_TOPK:
            key = softmax(s) + b
        elif mode == TOPK_THEN_SOFTMAX:
            key = s + b
        elif mode == SIGMOID_THEN_TOPK:
            key = sigmoid(s) + b
        else:
            raise ValueError(f"unknown score mode {mode}")
    return key.astype(np.float32)


def top_k(scores: np.ndarray, k: int):
    """The k experts with the highest scores per token ([MIN] Router: logits.topk;
    [RS] the MoE listing: topk over the scores).  Ties go to the lower expert
    index; slot j holds the j-th best.  Also returns near_tie[t] = 1 when the
    gap between the k-th and (k+1)-th best scores is below 1e-4 (0 when k = E)."""
    scores = np.asarray(scores, np.float32)
    T, E = scores.shape
    order = np.argsort(-scores, axis=1, kind="stable")     # descending; stable keeps lower index first
    idx = order[:, :k].astype(np.int32)
    near = np.zeros(T, np.int32)
    if k < E:
        kth = np.take_along_axis(scores, order[:, k - 1:k], axis=1)[:, 0].astype(np.float64)
        nxt = np.take_along_axis(scores, order[:, k:k + 1], axis=1)[:, 0].astype(np.float64)
        near = (kth - nxt < NEAR_TIE_GAP).astype(np.int32)
    return idx, near


def gate_weights(scores: np.ndarray, idx: np.ndarray, mode: int, renorm: bool) -> np.ndarray:
    """Combination weights of the chosen experts, float32.

    SOFTMAX_THEN_TOPK: p = softmax over all E scores and w_j = p of the j-th
    chosen expert ([TM] 17.2: Switch and Qwen2 keep the K largest of a full
    softmax); with renorm, w_j = p_j / sum over the chosen p ([RS] "The router"
    equation and worked example).
    TOPK_THEN_SOFTMAX: w = softmax over the chosen k scores alone ([TM] 17.2,
    Mixtral; [MIN] Router; [LT] gate equation).
    SIGMOID_THEN_TOPK: g = sigmoid(s) per expert and w_j = g_j / sum over the
    chosen g ([RS] "The router": DeepSeek-V3 scores with a sigmoid, normalized
    over the chosen experts); renorm does not apply.
    The weights use the scores only: a selection bias never enters them."""
    s = np.asarray(scores, np.float64)
    ii = idx.astype(np.int64)
    if mode == SOFTMAX_THEN_TOPK:
        p = softmax(s)
        w = np.take_along_axis(p, ii, axis=1)
        if renorm:
            w = w / w.sum(axis=1, keepdims=True)
    elif mode == TOPK_THEN_SOFTMAX:
        w = softmax(np.take_along_axis(s, ii, axis=1))
    elif mode == SIGMOID_THEN_TOPK:
        g = np.take_along_axis(sigmoid(s), ii, axis=1)
        w = g / g.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown score mode {mode}")
    return w.astype(np.float32)


def route(x, w_router, bias, k: int, mode: int, renorm: bool, select_bias=None):
    """Router step: (scores[T][E] f32, idx[T][k] i32, w[T][k] f32, near_tie[T] i32).
    near_tie refers to the selection keys (selection_keys)."""
    s = router_scores(x, w_router, bias)
    idx, near = top_k(selection_keys(s, mode, select_bias), k)
    return s, idx, gate_weights(s, idx, mode, renorm), near


def bias_update(select_bias: np.ndarray, counts: np.ndarray, T: int, k: int, rate: float) -> np.ndarray:
    """One step of bias balancing ([RS] "Keeping the load even", and the MoE
    listing's update after each step): raise b_e by a fixed amount when expert e
    got fewer than its share of the T k assignments, lower it when it got more,
    leave it when it got exactly its share.  f_e = counts_e / (T k) is compared
    with 1/E exactly (as integers: T k against E counts_e); the update is the
    float32 sum b_e + rate * sign, as the listing's float32 buffer computes it."""
    b = np.asarray(select_bias, np.float32)
    counts = np.asarray(counts, np.int64)
    E = b.shape[0]
    sign = np.sign(np.int64(T) * k - E * counts).astype(np.float32)
    return (b + np.float32(rate) * sign).astype(np.float32)


# ----------------------------------------------------------------------------
# Capacity and dispatch.

def capacity(T: int, k: int, E: int, phi: Optional[float]) -> Optional[int]:
    """C = ceil(phi * k * T / E) ([TM] 17.5 equation; [UD] "Capacity": T k / E is
    each expert's even share and phi the buffer over it).  phi is taken as the
    exact rational value of the given float; None means dropless (no cap)."""
    if phi is None:
        return None
    return math.ceil(Fraction(phi) * T * k / E)


def dispatch(idx: np.ndarray, E: int, cap: Optional[int]):
    """Group the (token, slot) assignments by expert ([MIN] MoELayer and [RS]
    the MoE listing: for each expert, the (token, slot) pairs that chose it).

    Tokens reach their experts in ascending token order; an expert that already
    holds cap tokens drops later arrivals ([MIN] "Capacity factor": tokens
    arriving at a full expert are dropped; [UD] "Capacity").

    Returns counts[E] (demand, before the cap), offsets[E+1] (exclusive scan of
    the kept counts), row_of[T][k] (row of the assignment in the permuted
    order, -1 when dropped) and perm_token[R] (token of each permuted row)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    rank = np.zeros((T, k), np.int64)
    for t in range(T):                       # one pass in arrival (token) order
        for j in range(k):
            e = idx[t, j]
            rank[t, j] = counts[e]
            counts[e] += 1
    kept = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of = np.full((T, k), -1, np.int64)
    perm_token = np.zeros(int(offsets[E]), np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if cap is None or rank[t, j] < cap:
                r = offsets[e] + rank[t, j]
                row_of[t, j] = r
                perm_token[r] = t
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_of.astype(np.int32), perm_token.astype(np.int32))


def dispatch_padded(idx: np.ndarray, E: int, cap: int):
    """The same dispatch in a capacity-padded layout: every expert owns C = cap
    slots, expert e's r-th kept assignment sits in slot e C + r, and the slots
    past its kept count are padding ([TM] 17.5: each expert processes at most C
    tokens in a fixed-size buffer; [UD] "Capacity"; [RS] "What experts cost at
    serving time": the buffers an expert-parallel exchange sends).

    Returns counts[E] (demand), offsets[E+1] = e C, row_of[T][k] (slot, -1 when
    dropped) and slot_token[E C] (token of each slot, -1 for padding)."""
    if cap is None or cap < 1:
        raise ValueError("the padded layout needs a capacity of at least 1")
    counts, offsets, row_of, perm_token = dispatch(idx, E, cap)
    kept = np.diff(offsets).astype(np.int64)
    slot_token = np.full(E * cap, -1, np.int64)
    row_pad = np.full(row_of.shape, -1, np.int64)
    for e in range(E):
        for r in range(int(kept[e])):
            slot_token[e * cap + r] = perm_token[offsets[e] + r]
    for t in range(row_of.shape[0]):
        for j in range(row_of.shape[1]):
            r = int(row_of[t, j])
            if r >= 0:
                e = int(idx[t, j])
                row_pad[t, j] = e * cap + (r - int(offsets[e]))
    return (counts, (np.arange(E + 1, dtype=np.int64) * cap).astype(np.int32),
            row_pad.astype(np.int32), slot_token.astype(np.int32))


def gather_slots(x: np.ndarray, slot_token: np.ndarray) -> np.ndarray:
    """x_slots[s] = x[slot_token[s]], zeros for padding slots (token -1)."""
    x = np.asarray(x)
    st = np.asarray(slot_token, np.int64)
    out = np.zeros((st.shape[0], x.shape[1]), x.dtype)
    out[st >= 0] = x[st[st >= 0]]
    return out


def permute_rows(x: np.ndarray, perm_token: np.ndarray) -> np.ndarray:
    """x_perm[r] = x[perm_token[r]] ([MIN] x_flat[tok]; [RS] x[rows])."""
    return np.asarray(x)[np.asarray(perm_token, np.int64)]


# ----------------------------------------------------------------------------
# Experts.

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), float64."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_hidden(h, w_gate, w_up) -> np.ndarray:
    """a = SiLU(h gate^T) * (h up^T) ([RS] the MoE listing, F.silu(h @ gate[e]) * (h @ up[e]),
    with the weights held (F, d) here), float64."""
    h = np.asarray(h, np.float64)
    return silu(h @ np.asarray(w_gate, np.float64).T) * (h @ np.asarray(w_up, np.float64).T)


def swiglu(h, w_gate, w_up, w_down) -> np.ndarray:
    """A SwiGLU expert: (SiLU(h Wg) * (h Wu)) Wd ([RS] "The router": each expert an
    ordinary SwiGLU MLP; the MoE listing), float64, down held (d, F)."""
    return swiglu_hidden(h, w_gate, w_up) @ np.asarray(w_down, np.float64).T


def grouped_swiglu(x_perm, offsets, expert_weights):
    """Run expert e on its rows [offsets[e], offsets[e+1]) ([RS] the MoE listing's
    per-expert loop; [MIN] "Capacity factor": dropless routing as a variable-size
    grouped GEMM).  expert_weights(e) -> (gate, up, down).  Returns the hidden
    activations a[R][F] and outputs y_perm[R][d], float64."""
    offsets = np.asarray(offsets, np.int64)
    R = int(offsets[-1])
    a = y = None
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        g, u, dn = expert_weights(e)
        ae = swiglu_hidden(np.asarray(x_perm[lo:hi]), g, u)
        ye = ae @ np.asarray(dn, np.float64).T
        if a is None:
            a = np.zeros((R, ae.shape[1]), np.float64)
            y = np.zeros((R, ye.shape[1]), np.float64)
        a[lo:hi], y[lo:hi] = ae, ye
    return a, y


# ----------------------------------------------------------------------------
# Combine.

def combine(y_perm, row_of, w, shared_out=None, d: Optional[int] = None) -> np.ndarray:
    """y[t] = sum over kept slots j of w[t][j] * y_perm[row_of[t][j]], plus the
    shared expert's output, unweighted ([TM] 17.2 equation; [MIN] out[tok] +=
    weights * expert(x), then out += shared(x); [RS] index_add_ of y * weight).
    A dropped slot adds nothing ([TM] 17.5).  float64."""
    row_of = np.asarray(row_of, np.int64)
    T, k = row_of.shape
    if d is None:
        d = np.asarray(y_perm).shape[1] if shared_out is None else np.asarray(shared_out).shape[1]
    y = np.zeros((T, d), np.float64) if shared_out is None else np.array(shared_out, np.float64)
    w = np.asarray(w, np.float64)
    for j in range(k):
        kept = row_of[:, j] >= 0
        if kept.any():
            y[kept] += w[kept, j][:, None] * np.asarray(y_perm, np.float64)[row_of[kept, j]]
    return y


# ----------------------------------------------------------------------------
# Balance statistics.

def balance_stats(counts, scores, T: int, k: int, E: int, alpha: float):
    """f_i, P_i, L_aux and the demand max/mean load.

    f_i = counts_i / (T k): expert i's share of the token assignments ([RS] the
    MoE listing, counts / counts.sum(); [LT] "Keeping the load balanced"),
    as one float32 division.
    P_i = mean over tokens of the router's softmax probability of expert i
    ([MIN] load_balancing_loss; [RS] "Keeping the load even").
    L_aux = alpha * E * sum_i f_i P_i ([TM] 17.4 equation; [LT] balance equation).
    max/mean = E * max_i counts_i / (T k), the demand-side load of the busiest
    expert over the mean ([UD] "Load imbalance"), as one float32 division.
    Returns (f f32[E], P f32[E], L_aux f32, max_over_mean f32)."""
    counts = np.asarray(counts, np.int64)
    tk = np.float32(T * k)
    f = (counts.astype(np.float32) / tk).astype(np.float32)
    P = softmax(scores).mean(axis=0)
    l_aux = alpha * E * float(np.sum(f.astype(np.float64) * P))
    mom = np.float32(np.float32(E * int(counts.max())) / tk)
    return f, P.astype(np.float32), np.float32(l_aux), mom


# ----------------------------------------------------------------------------
# Whole layer.

def layer_forward(x, w_router, bias, expert_weights, shared_weights, *, k: int, mode: int,
                  renorm: bool, phi: Optional[float], alpha: float, dtype: str, select_bias=None,
                  timings: Optional[dict] = None):
    """The full layer, step by step, returning every intermediate.

    x, w_router: stored values (float32 arrays).  expert_weights(e) ->
    (gate[F][d], up[F][d], down[d][F]); shared_weights: the same triple or None.
    dtype: "bf16" or "f32", the output storage type of y.
    timings: if a dict is given, the wall seconds of each step are stored in it
    (route, dispatch, experts, shared_expert, combine, stats)."""
    import time
    clock = [time.perf_counter()]

    def lap(name):
        now = time.perf_counter()
        if timings is not None:
            timings[name] = now - clock[0]
        clock[0] = now

    x = np.asarray(x, np.float32)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    s, idx, w, near = route(x, w_router, bias, k, mode, renorm, select_bias)
    lap("route")
    cap = capacity(T, k, E, phi)
    counts, offsets, row_of, perm_token = dispatch(idx, E, cap)
    x_perm = permute_rows(x, perm_token)
    lap("dispatch")
    a, y_perm = grouped_swiglu(x_perm, offsets, expert_weights)
    lap("experts")
    shared = None if shared_weights is None else swiglu(x, *shared_weights)
    lap("shared_expert")
    y64 = combine(y_perm, row_of, w, shared, d=x.shape[1])
    y = round_to(y64, dtype)
    lap("combine")
    f, P, l_aux, mom = balance_stats(counts, s, T, k, E, alpha)
    lap("stats")
    return dict(scores=s, idx=idx, w=w, near_tie=near, capacity=cap, counts=counts,
                offsets=offsets, row_of=row_of, perm_token=perm_token, x_perm=x_perm,
                a=a, y_perm=y_perm, shared=shared, y64=y64, y=y,
                f=f, P=P, l_aux=l_aux, max_over_mean=mom)


def token_output(x_t, idx_t, w_t, kept_t, expert_weights, shared_weights=None) -> np.ndarray:
    """y for one token straight from the definition, without any permutation:
    sum over its kept slots of w * Expert(x) plus the shared expert ([TM] 17.2
    equation; [MIN] MoELayer loop).  float64."""
    x_t = np.asarray(x_t, np.float64)[None, :]
    y = np.zeros(x_t.shape[1], np.float64)
    for e, wj, kj in zip(idx_t, w_t, kept_t):
        if kj:
            y += float(wj) * swiglu(x_t, *expert_weights(int(e)))[0]
    if shared_weights is not None:
        y += swiglu(x_t, *shared_weights)[0]
    return y


def experts_touched_expected(E: int, k: int, B: int) -> float:
    """Expected number of distinct experts a batch of B tokens touches when each
    picks k of E uniformly: E (1 - (1 - k/E)^B) ([RS] "Counting real models")."""
    return E * (1.0 - (1.0 - k / E) ** B)
