"""Pins of the oracle's quantised expert pass (forward and backward) against a brute-force
implementation that spells out every MXFP8 quantisation block by block.

The brute force has its own scalar e4m3 encoder (nearest of the 127 non-negative finite codes
by exhaustive search, ties to the even code) and its own block scale (floor(log2 amax) - 8 from
math.frexp), and it states each quantisation axis as explicit index loops: weights along their
GEMM's reduction axis (W1 along d, W2 along I), the transposed weights along the dgrad GEMMs'
(W2^T along d, W1^T along 2I), h along I, [dG dU] along 2I, and the weight-gradient operands
along tokens (32-row blocks from the expert's first row, zero tail).  The inputs scale rows and
columns of every matrix by different powers of two, so quantising any tensor along the other
axis changes the result; a test below checks that a swapped axis is detected.
"""
import math

import numpy as np
import pytest

import moe_inputs
import oracle
from oracle.layer import _qdq

# ---------------------------------------------------------------- brute-force MXFP8


def _e4m3_value(c):
    e, m = (c >> 3) & 15, c & 7
    return (1 + m / 8.0) * 2.0 ** (e - 7) if e else m * 2.0 ** -9


_VALUES = [_e4m3_value(c) for c in range(127)]   # codes 0x00 .. 0x7E (0x7F is NaN)


def _nearest(x):
    """e4m3 value nearest to |x| <= 448 (ties to the even code), with the sign of x."""
    a = abs(x)
    best, bd = 0, None
    for c, v in enumerate(_VALUES):
        dd = abs(v - a)
        if bd is None or dd < bd or (dd == bd and c % 2 == 0):
            best, bd = c, dd
    return math.copysign(_VALUES[best], x)


def _qdq_block(vals):
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return [0.0] * len(vals)
    e = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
    s = 2.0 ** e
    return [_nearest(max(-448.0, min(448.0, v / s))) * s for v in vals]


def qdq_rows(M):
    """Every row quantised in blocks of 32 consecutive columns."""
    M = np.asarray(M, dtype=np.float64)
    out = np.empty_like(M)
    for i in range(M.shape[0]):
        for b in range(0, M.shape[1], 32):
            out[i, b:b + 32] = _qdq_block(list(M[i, b:b + 32]))
    return out


def qdq_cols(M):
    """Every column quantised in blocks of 32 consecutive rows (a zero tail pads the last block)."""
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[0]
    out = np.empty_like(M)
    for j in range(M.shape[1]):
        for b in range(0, n, 32):
            blk = list(M[b:b + 32, j]) + [0.0] * max(0, b + 32 - n)
            out[b:b + 32, j] = _qdq_block(blk)[:min(32, n - b)]
    return out


def f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def brute_expert(A, w1, w2, DY, wrow, swap=None):
    """Quantised expert forward + backward written out with explicit block loops.
    swap: name of one tensor to quantise along the wrong axis (to show the inputs detect it)."""
    q = {"W1": qdq_rows, "W2": qdq_rows, "H": qdq_rows, "W2t": qdq_cols, "W1t": qdq_cols, "DGU": qdq_rows,
         "tok": qdq_cols}
    if swap:
        q[swap] = qdq_cols if q[swap] is qdq_rows else qdq_rows
    I = w1.shape[0] // 2
    W1 = q["W1"](w1)                      # [2I, d], blocks along d
    W2 = q["W2"](w2)                      # [d, I], blocks along I
    G = np.einsum("nk,ik->ni", A, W1[:I])
    U = np.einsum("nk,ik->ni", A, W1[I:])
    h = f32(G / (1.0 + np.exp(-G)) * U)
    H = q["H"](h)                         # blocks along I
    Y = np.einsum("ni,di->nd", H, W2)
    W2t = q["W2t"](W2)                    # [d, I], blocks along d
    W1t = q["W1t"](W1)                    # [2I, d], blocks along 2I
    dH = wrow[:, None] * np.einsum("nd,di->ni", DY, W2t)
    s = 1.0 / (1.0 + np.exp(-G))
    dGU = f32(np.concatenate([dH * U * s * (1.0 + G * (1.0 - s)), dH * G * s], axis=1))
    DGU = q["DGU"](dGU)                   # blocks along 2I
    dX = np.einsum("nj,jd->nd", DGU, W1t)
    dYw = f32(f32(wrow)[:, None] * DY)
    dW2 = np.einsum("nd,ni->di", q["tok"](dYw), q["tok"](H))
    dW1 = np.einsum("nj,nd->jd", q["tok"](DGU), q["tok"](A))
    return dict(G=G, U=U, H=H, Y=Y, DGU=DGU, dX=dX, dW1=dW1, dW2=dW2)


# ---------------------------------------------------------------- inputs


def _inputs(n=40, d=64, I=32, seed=31):
    rng = np.random.default_rng(seed)

    def scaled(shape, lo, hi):
        a = rng.standard_normal(shape)
        a *= np.exp2(rng.integers(lo, hi, size=(shape[0], 1)))   # row scales
        a *= np.exp2(rng.integers(lo, hi, size=(1, shape[1])))   # column scales
        return a.astype(np.float32)

    A = oracle.dequantize(*oracle.quantize(scaled((n, d), -3, 4).astype(np.float64), axis=1), axis=1)
    w1 = scaled((2 * I, d), -6, 1) / 8
    w2 = scaled((d, I), -6, 1) / 8
    DY = oracle.dequantize(*oracle.quantize(scaled((n, d), -3, 4).astype(np.float64), axis=1), axis=1)
    wrow = rng.uniform(0.05, 1.0, n)
    return A, w1, w2, DY, wrow


def _close(a, b, tol=1e-10):
    scale = np.max(np.abs(b)) + 1e-300
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) <= tol * scale


@pytest.fixture(scope="module")
def case():
    A, w1, w2, DY, wrow = _inputs()
    return A, w1, w2, DY, wrow, brute_expert(A, w1, w2, DY, wrow)


def test_brute_encoder_agrees_with_oracle_codec():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(300) * np.exp2(rng.integers(-12, 9, 300))
    v = np.clip(v, -448, 448)
    assert np.array_equal(np.array([_nearest(x) for x in v]), oracle.e4m3_decode(oracle.e4m3_encode(v)))


def test_oracle_experts_quantise_weights_along_the_reduction_axes(case):
    A, w1, w2, DY, wrow, ref = case
    W1, W2 = oracle.oracle_experts([w1], [w2])(0)
    assert np.array_equal(W1, qdq_rows(w1)) and np.array_equal(W2, qdq_rows(w2))
    assert not np.array_equal(W1, qdq_cols(w1)) and not np.array_equal(W2, qdq_cols(w2))


def test_quantised_expert_forward_and_backward_match_brute_force(case):
    A, w1, w2, DY, wrow, ref = case
    W1, W2 = oracle.oracle_experts([w1], [w2])(0)
    fe = oracle.expert_forward(A, W1, W2)
    assert _close(fe.G, ref["G"]) and _close(fe.U, ref["U"])
    assert np.array_equal(fe.H, ref["H"])
    assert _close(fe.Y, ref["Y"])
    be = oracle.expert_backward(fe, A, DY, wrow, _qdq(W1, 0, True)[2], _qdq(W2, 0, True)[2])
    assert np.array_equal(be.DGU, ref["DGU"])
    assert _close(be.dX, ref["dX"]) and _close(be.dW1, ref["dW1"]) and _close(be.dW2, ref["dW2"])


def test_layer_backward_requantises_along_the_brute_force_axes():
    """One expert, top-1: the layer's own choice of axes for W2^T, W1^T, [dG dU] and the token-axis
    operands equals the brute force (dx rows, dW1, dW2)."""
    cfg = moe_inputs.LayerConfig("one", T=40, d=64, E=1, k=1, inter=32, score="softmax", seed=32)
    A, w1, w2, DY, _ = _inputs(seed=33)
    x = moe_inputs.bf16_values(moe_inputs.bf16_bits(A.astype(np.float32))).astype(np.float64)
    dy = moe_inputs.bf16_values(moe_inputs.bf16_bits(DY.astype(np.float32))).astype(np.float64)
    w_r = np.ones((1, 64)) * 2.0 ** -6
    ex = oracle.oracle_experts([w1], [w2])
    fw = oracle.layer_forward(x, w_r, ex, 1, "softmax")
    bw = oracle.layer_backward(fw, dy, x, w_r, ex, "softmax")
    X = oracle.dequantize(*oracle.quantize(x, axis=1), axis=1)
    DYq = oracle.dequantize(*oracle.quantize(dy, axis=1), axis=1)
    ref = brute_expert(X, w1, w2, DYq, np.ones(40))
    assert _close(fw.y, ref["Y"])
    assert _close(bw.dx, ref["dX"])          # k = 1 softmax: the router term is exactly zero
    assert _close(bw.dW1[0], ref["dW1"]) and _close(bw.dW2[0], ref["dW2"])


@pytest.mark.parametrize("swap", ["W1", "W2", "H", "W2t", "W1t", "DGU", "tok"])
def test_inputs_detect_a_swapped_axis(case, swap):
    """Quantising any one tensor along the other axis changes a compared result."""
    A, w1, w2, DY, wrow, ref = case
    bad = brute_expert(A, w1, w2, DY, wrow, swap=swap)
    differs = [k for k in ref if not _close(bad[k], ref[k], tol=1e-12)]
    assert differs, swap
