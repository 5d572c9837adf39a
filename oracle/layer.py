"""Reference MoE layer: router, top-k, schedule, MXFP8 SwiGLU experts, combine, backward.

Test infrastructure (see the package docstring).  The pages describe the layer
only in words: a router picks a few experts per token, tokens are dispatched to
the experts, each expert runs its FFN, the results are gathered back and
combined (commentary "Cursor 开源 MoK…", section 什么是MoK; article "Cursor 為
Composer 改造 MoE 訓練…", opening section); the layer is DeepSeek-V3-style and
computed in MXFP8 (knowledge card, section 方法/产品要点); the schedule built
in the forward pass is reused by the backward pass, whose directions are
reverse-combine then reverse-dispatch (same section).  MoK reaches the plain
layer result, fused and deterministic (knowledge card, 一句话结论), so this
module is the plain definition written out in float64.

Everything the pages leave open is a reading stated where it is taken:
the router is a plain linear map (plus an optional per-expert bias), the expert
FFN is SwiGLU with gate rows first, top-k ties go to the lower expert index and
slot j of a token is its j-th best expert, GEMM operands are MXFP8 quantised
along each GEMM's reduction axis, and the backward pass is straight-through
(quantisation acts as the identity in the gradient).

``quant=False`` replaces every quantise/dequantise pair by the identity; that
unquantised layer is smooth in its inputs and is what the finite-difference
pins differentiate.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .mxfp8 import BLOCK, dequantize, quantize

# ----------------------------------------------------------------------------
# helpers


def _f32(a: np.ndarray) -> np.ndarray:
    """Round to the nearest float32 value (kept in float64)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _qdq(a: np.ndarray, axis: int, quant: bool):
    """(codes, scales, dequantised values) of ``a`` quantised along ``axis``; identity if not quant."""
    if not quant:
        return None, None, np.asarray(a, dtype=np.float64)
    q, s = quantize(a, axis=axis)
    return q, s, dequantize(q, s, axis=axis)


def token_quantize(a: np.ndarray):
    """MXFP8 codes and scales of one expert's rows quantised along the token axis (axis 0).

    Reading of "requantisation of transposed operands" for the weight-gradient
    GEMMs, whose reduction axis is the token axis: blocks of 32 consecutive rows
    start at the first row of the expert's segment, and a ragged tail is padded
    with zero rows (zeros change neither a block maximum nor a sum).  Returns
    (codes [npad, ...], scales [npad / 32, ...]) with npad = n rounded up to 32.
    """
    a = np.asarray(a, dtype=np.float64)
    n = a.shape[0]
    npad = -(-n // BLOCK) * BLOCK
    padded = np.zeros((npad,) + a.shape[1:], dtype=np.float64)
    padded[:n] = a
    return quantize(padded, axis=0)


def token_requant(a: np.ndarray, quant: bool = True) -> np.ndarray:
    """One expert's rows requantised along the token axis (``token_quantize``), dequantised."""
    a = np.asarray(a, dtype=np.float64)
    if not quant:
        return a
    q, s = token_quantize(a)
    return dequantize(q, s, axis=0)[: a.shape[0]]


def swiglu(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """h = silu(G) U = G sigmoid(G) U (the expert's gated activation)."""
    G = np.asarray(G, dtype=np.float64)
    return G * _sigmoid(G) * np.asarray(U, dtype=np.float64)


def swiglu_backward(dH: np.ndarray, G: np.ndarray, U: np.ndarray):
    """(dG, dU) of h = silu(G) U for upstream dH: with s = sigmoid(G),
    dG = dH U s (1 + G (1 - s)) and dU = dH G s."""
    G = np.asarray(G, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    s = _sigmoid(G)
    return dH * U * s * (1.0 + G * (1.0 - s)), dH * G * s


# ----------------------------------------------------------------------------
# router, selection, weights, schedule


def router_logits(x: np.ndarray, w_r: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Router logits L = x W_r^T (+ bias), float64.

    The pages say only that a router picks a few experts per token (article
    "Cursor 為 Composer 改造 MoE 訓練…", opening section).  Reading: a linear
    router over the bf16 activations, as in DeepSeek-V3-style layers, with an
    optional per-expert bias added to every token's logits.
    """
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """idx[t, j] = the j-th best expert of token t (int32 [T, k]).

    The selection is decided on float32 logits (the precision the kernel holds
    them in), best first, equal logits ordered by increasing expert index.
    Selecting on logits equals selecting on softmax or sigmoid scores, both
    being increasing functions of the logit.
    """
    L32 = np.asarray(L, dtype=np.float64).astype(np.float32)
    order = np.argsort(-L32, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def routing_weights(L: np.ndarray, idx: np.ndarray, score: str) -> np.ndarray:
    """Combine weights w[t, j] of the selected experts (float64 [T, k]).

    "softmax": softmax over the k selected logits, which equals the full
    softmax renormalised over the selection.  "sigmoid": per-expert sigmoid
    scores of the selected experts divided by their sum (DeepSeek-V3 style,
    without its selection bias, group limit or routed scaling factor, none of
    which the workloads name).
    """
    Ls = np.take_along_axis(np.asarray(L, dtype=np.float64), idx.astype(np.int64), axis=1)
    if score == "softmax":
        z = np.exp(Ls - Ls[:, :1])  # Ls[:, 0] is the largest selected logit
        return z / z.sum(axis=1, keepdims=True)
    if score == "sigmoid":
        s = _sigmoid(Ls)
        return s / s.sum(axis=1, keepdims=True)
    raise ValueError(score)


@dataclass
class Schedule:
    counts: np.ndarray       # [E] int64 rows per expert
    offsets: np.ndarray      # [E+1] exclusive prefix sum of counts
    padded_offsets: np.ndarray  # [E+1] prefix sum of counts rounded up to 32
    perm: np.ndarray         # [T*k] slot id t*k+j of permuted row r
    pos: np.ndarray          # [T, k] permuted row of slot (t, j)


def build_schedule(idx: np.ndarray, E: int) -> Schedule:
    """Expert-major stable permutation of the T*k routed slots.

    The pages' schedule is built on the device once and reused by the backward
    pass (knowledge card, 方法/产品要点).  Reading of what it holds: permuted
    row r lists the slots of expert 0 first, then expert 1, ...; within an
    expert the slots keep increasing token order (a token selects an expert at
    most once).  pos is the inverse map.  Padded offsets round every expert's
    row count up to a multiple of 32 (one MXFP8 block along the token axis).
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    padded = np.concatenate([[0], np.cumsum(-(-counts // BLOCK) * BLOCK)]).astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    pos = np.empty(T * k, dtype=np.int64)
    pos[perm] = np.arange(T * k)
    return Schedule(counts, offsets, padded, perm, pos.reshape(T, k))


# ----------------------------------------------------------------------------
# experts


@dataclass
class ExpertForward:
    G: np.ndarray      # [n, I] gate pre-activations
    U: np.ndarray      # [n, I] up projections
    h: np.ndarray      # [n, I] silu(G) * U rounded to float32
    Hq: np.ndarray | None
    Hs: np.ndarray | None
    H: np.ndarray      # [n, I] dequantised h (the down GEMM's operand)
    Y: np.ndarray      # [n, d] expert output rows


def expert_forward(A: np.ndarray, W1: np.ndarray, W2: np.ndarray, quant: bool = True) -> ExpertForward:
    """SwiGLU expert on dispatched rows: G = A W1g^T, U = A W1u^T, h = silu(G) U, Y = Q(h) W2^T.

    ``A`` are the (dequantised) rows routed to the expert, ``W1`` [2I, d] holds
    the gate rows then the up rows, ``W2`` is [d, I]; both dequantised.  The
    kernel quantises h from float32 values, so h is rounded to float32 before
    it is quantised along I.
    """
    I = W1.shape[0] // 2
    G = A @ W1[:I].T
    U = A @ W1[I:].T
    h = swiglu(G, U)
    if quant:
        h = _f32(h)
    Hq, Hs, H = _qdq(h, 1, quant)
    Y = H @ W2.T
    return ExpertForward(G, U, h, Hq, Hs, H, Y)


@dataclass
class ExpertBackward:
    dH: np.ndarray     # [n, I]
    dGU: np.ndarray    # [n, 2I] float32-rounded [dG dU] before quantisation
    dGUq: np.ndarray | None
    dGUs: np.ndarray | None
    DGU: np.ndarray    # [n, 2I] dequantised
    dX: np.ndarray     # [n, d] input-gradient rows
    dW1: np.ndarray    # [2I, d]
    dW2: np.ndarray    # [d, I]


def expert_backward(fw: ExpertForward, A: np.ndarray, DYrows: np.ndarray, wrow: np.ndarray,
                    W1t: np.ndarray, W2t: np.ndarray, quant: bool = True) -> ExpertBackward:
    """Backward of one expert (straight-through through every quantiser).

    ``DYrows`` [n, d] are the dequantised upstream-gradient rows of the
    expert's tokens, ``wrow`` [n] their combine weights, ``W2t`` [d, I] and
    ``W1t`` [2I, d] the expert weights requantised along d and 2I (the dgrad
    GEMMs' reduction axes).

    * dH = w * (dY W2)                      (dgrad of the down GEMM)
    * dG = dH U s (1 + G (1 - s)), dU = dH G s, with s = sigmoid(G)
    * [dG dU] rounded to float32 and quantised along 2I
    * dX = [dG dU] W1                        (dgrad of the gate/up GEMM)
    * dW2 = Q_tok(w * dY)^T Q_tok(H),  dW1 = Q_tok([dG dU])^T Q_tok(A)
      where Q_tok requantises along the token axis (``token_requant``) and
      w * dY is rounded to float32 from a float32 weight (the kernel's
      precision for that decision).
    """
    dH = wrow[:, None] * (DYrows @ W2t)
    dG, dU = swiglu_backward(dH, fw.G, fw.U)
    dGU = np.concatenate([dG, dU], axis=1)
    if quant:
        dGU = _f32(dGU)
    dGUq, dGUs, DGU = _qdq(dGU, 1, quant)
    dX = DGU @ W1t
    w32 = _f32(wrow) if quant else wrow
    dYw = _f32(w32[:, None] * DYrows) if quant else wrow[:, None] * DYrows
    dW2 = token_requant(dYw, quant).T @ token_requant(fw.H, quant)
    dW1 = token_requant(DGU, quant).T @ token_requant(A, quant)
    return ExpertBackward(dH, dGU, dGUq, dGUs, DGU, dX, dW1, dW2)


# ----------------------------------------------------------------------------
# whole layer


def oracle_experts(w1_list, w2_list, quant: bool = True):
    """Dequantised per-expert weights as the layer sees them.

    Returns a function e -> (W1 [2I, d] quantised along d, W2 [d, I] quantised
    along I) built from float32 weights (each GEMM's reduction axis).
    """
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = (_qdq(w1_list[e], 1, quant)[2], _qdq(w2_list[e], 1, quant)[2])
        return cache[e]

    return get


@dataclass
class LayerForward:
    L: np.ndarray
    idx: np.ndarray
    w: np.ndarray
    sched: Schedule
    xq: np.ndarray | None
    xs: np.ndarray | None
    X: np.ndarray              # [T, d] dequantised x
    experts: dict              # e -> ExpertForward (rows in schedule order)
    rows_of: dict              # e -> token index of each row of the expert
    Yrows: np.ndarray          # [T*k + S*T, d] expert outputs in permuted-row order
    y: np.ndarray              # [T, d] float64 layer output
    n_shared: int


def combine(Yrows: np.ndarray, w: np.ndarray, pos: np.ndarray, n_shared: int = 0) -> np.ndarray:
    """y[t] = sum_j w[t, j] Y[pos[t, j]] (+ the shared expert's row of t, weight 1).

    Results are pushed back to their tokens and summed in the fixed slot order
    j = 0..k-1, then the shared expert (push-based combine: knowledge card,
    方法/产品要点).
    """
    T, k = w.shape
    y = np.zeros((T, Yrows.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * Yrows[pos[:, j]]
    for s in range(n_shared):
        y += Yrows[T * k + s * T: T * k + (s + 1) * T]
    return y


def layer_forward(x, w_r, experts, k: int, score: str, bias=None, n_shared: int = 0,
                  quant: bool = True) -> LayerForward:
    """The layer's forward pass: route, dispatch rows to experts, SwiGLU FFN, combine.

    ``experts(e)`` returns dequantised (W1 [2I, d], W2 [d, I]); e == E is the
    shared expert, which sees every token with weight 1.
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    E = np.asarray(w_r).shape[0]
    L = router_logits(x, w_r, bias)
    idx = select_topk(L, k)
    w = routing_weights(L, idx, score)
    sched = build_schedule(idx, E)
    xq, xs, X = _qdq(x, 1, quant)
    R = T * k
    Yrows = np.zeros((R + n_shared * T, d), dtype=np.float64)
    outs, rows_of = {}, {}
    for e in range(E + n_shared):
        if e < E:
            lo, hi = sched.offsets[e], sched.offsets[e + 1]
            tokens = sched.perm[lo:hi] // k
        else:
            lo, hi = R + (e - E) * T, R + (e - E + 1) * T
            tokens = np.arange(T)
        rows_of[e] = tokens
        if hi == lo:
            continue
        W1, W2 = experts(e)
        fw = expert_forward(X[tokens], W1, W2, quant)
        outs[e] = fw
        Yrows[lo:hi] = fw.Y
    y = combine(Yrows, w, sched.pos, n_shared)
    return LayerForward(L, idx, w, sched, xq, xs, X, outs, rows_of, Yrows, y, n_shared)


def router_backward(L: np.ndarray, idx: np.ndarray, w: np.ndarray, dw: np.ndarray, score: str) -> np.ndarray:
    """Gradient of the loss with respect to the selected logits, [T, k].

    softmax over the selection: dL_j = w_j (dw_j - sum_i w_i dw_i).
    normalised sigmoid: with s = sigmoid(L), w = s / sum s,
    dL_j = s_j (1 - s_j) (dw_j - sum_i w_i dw_i) / sum_i s_i.
    Unselected experts receive no gradient (the selection is piecewise constant).
    """
    inner = np.sum(w * dw, axis=1, keepdims=True)
    if score == "softmax":
        return w * (dw - inner)
    Ls = np.take_along_axis(np.asarray(L, dtype=np.float64), idx.astype(np.int64), axis=1)
    s = _sigmoid(Ls)
    return s * (1.0 - s) * (dw - inner) / s.sum(axis=1, keepdims=True)


@dataclass
class LayerBackward:
    dyq: np.ndarray | None
    dys: np.ndarray | None
    dw: np.ndarray          # [T, k] gradient of the combine weights
    dL: np.ndarray          # [T, k] gradient of the selected logits
    dx: np.ndarray          # [T, d]
    dw_r: np.ndarray        # [E, d]
    dW1: dict               # e -> [2I, d]
    dW2: dict               # e -> [d, I]
    experts: dict           # e -> ExpertBackward
    dXrows: np.ndarray      # [T*k + S*T, d] input-gradient rows in permuted-row order


def layer_backward(fw: LayerForward, dy, x, w_r, experts, score: str, quant: bool = True,
                   expert_subset=None) -> LayerBackward:
    """The layer's backward pass for upstream gradient ``dy`` [T, d].

    Reverse-combine pulls each row's gradient from its token, the expert
    backward runs per expert, reverse-dispatch pushes input-gradient rows back
    to their tokens, where they are summed in slot order with the router's
    contribution (knowledge card, 方法/产品要点: pull reverse-combine, push
    reverse-dispatch, schedule reused from the forward pass).

    * dw[t, j] = <dy[t], Y[pos[t, j]]>     (combine weights; dy unquantised)
    * expert backward on DQ(Q(dy)) rows    (``expert_backward``)
    * dL from dw (``router_backward``); dW_r = dL^T x; the router adds dL W_r to dx
    * dx[t] = sum_j dX[pos[t, j]] + shared dX[t] + dL[t] W_r

    ``expert_subset`` limits the expert backward to some experts (dx and the
    router terms are then only partial); used to time a bounded sample.
    """
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    T, d = dy.shape
    k = fw.idx.shape[1]
    E = w_r.shape[0]
    R = T * k
    sched = fw.sched
    dyq, dys, DY = _qdq(dy, 1, quant)

    dw = np.empty((T, k), dtype=np.float64)
    for j in range(k):
        dw[:, j] = np.sum(dy * fw.Yrows[sched.pos[:, j]], axis=1)
    dLsel = router_backward(fw.L, fw.idx, fw.w, dw, score)
    dLfull = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dLfull, fw.idx.astype(np.int64), dLsel, axis=1)
    dw_r = dLfull.T @ x
    dx_router = dLfull @ w_r

    wflat = fw.w.reshape(-1)
    dXrows = np.zeros_like(fw.Yrows)
    outs, dW1, dW2 = {}, {}, {}
    todo = range(E + fw.n_shared) if expert_subset is None else expert_subset
    I = next(iter(fw.experts.values())).G.shape[1] if fw.experts else None
    for e in todo:
        if e not in fw.experts:
            if I is None:
                I = experts(e)[0].shape[0] // 2
            dW1[e] = np.zeros((2 * I, d))
            dW2[e] = np.zeros((d, I))
            continue
        W1, W2 = experts(e)
        tokens = fw.rows_of[e]
        if e < E:
            lo, hi = sched.offsets[e], sched.offsets[e + 1]
            wrow = wflat[sched.perm[lo:hi]]
        else:
            lo, hi = R + (e - E) * T, R + (e - E + 1) * T
            wrow = np.ones(T)
        W2t = _qdq(W2, 0, quant)[2]   # requantised along d
        W1t = _qdq(W1, 0, quant)[2]   # requantised along 2I
        bw = expert_backward(fw.experts[e], fw.X[tokens], DY[tokens], wrow, W1t, W2t, quant)
        outs[e] = bw
        dXrows[lo:hi] = bw.dX
        dW1[e] = bw.dW1
        dW2[e] = bw.dW2

    dx = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        dx += dXrows[sched.pos[:, j]]
    for s in range(fw.n_shared):
        dx += dXrows[R + s * T: R + (s + 1) * T]
    dx += dx_router
    return LayerBackward(dyq, dys, dw, dLsel, dx, dw_r, dW1, dW2, outs, dXrows)
