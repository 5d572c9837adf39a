"""Pins of the oracle's layer functions against brute force, closed forms and finite differences."""
import math
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs
import oracle


def _tiny(T=16, d=64, E=4, k=2, I=32, score="softmax", seed=11, n_shared=0, zipf=0.0):
    cfg = moe_inputs.LayerConfig("t", T=T, d=d, E=E, k=k, inter=I, score=score, seed=seed,
                                 n_shared=n_shared, zipf_s=zipf, zipf_lam=0.3)
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(E + n_shared)]
    return cfg, inp, ws


# ---------------------------------------------------------------- router / selection


def test_router_logits_exact_sums():
    cfg, inp, _ = _tiny(T=5, d=64, E=6)
    x, w_r = inp.x.astype(np.float64), inp.w_r.astype(np.float64)
    L = oracle.router_logits(x, w_r)
    for t in range(cfg.T):
        for e in range(cfg.E):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(w_r[e, i])) for i in range(cfg.d))
            assert abs(L[t, e] - float(exact)) <= 1e-13 * (1 + abs(float(exact)))


def test_router_bias_shifts_every_token():
    cfg, inp, _ = _tiny(T=3, E=5)
    b = np.arange(5, dtype=np.float64) * 0.25
    L0 = oracle.router_logits(inp.x, inp.w_r)
    L1 = oracle.router_logits(inp.x, inp.w_r, b)
    assert np.allclose(L1 - L0, b[None, :], atol=1e-15)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    L = rng.integers(-3, 4, size=(40, 7)).astype(np.float64)  # many exact ties
    for k in (1, 3, 7):
        idx = oracle.select_topk(L, k)
        for t in range(40):
            ref = sorted(range(7), key=lambda e: (-L[t, e], e))[:k]
            assert list(idx[t]) == ref


def test_topk_decided_in_float32():
    L = np.array([[1.0, 1.0 + 1e-12, 0.5]])  # equal once rounded to float32 -> lower index first
    assert list(oracle.select_topk(L, 2)[0]) == [0, 1]


def test_softmax_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((20, 9))
    idx = oracle.select_topk(L, 3)
    w = oracle.routing_weights(L, idx, "softmax")
    full = np.exp(L) / np.exp(L).sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-14)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)


def test_sigmoid_weights_special_cases():
    L = np.array([[2.0, 2.0, 2.0, -1.0], [0.0, 5.0, -5.0, 1.0]])
    idx = oracle.select_topk(L, 3)
    w = oracle.routing_weights(L, idx, "sigmoid")
    assert np.allclose(w[0], 1.0 / 3.0, atol=1e-15)
    assert np.all(np.diff(w[1]) <= 0)  # best expert first gets the largest weight
    s = 1 / (1 + math.exp(-5.0)), 1 / (1 + math.exp(-1.0)), 0.5
    assert np.allclose(w[1], np.array(s) / sum(s), rtol=1e-14)
    w1 = oracle.routing_weights(L, oracle.select_topk(L, 1), "sigmoid")
    assert np.all(w1 == 1.0)


# ---------------------------------------------------------------- schedule


def test_schedule_brute_force_and_invariants():
    rng = np.random.default_rng(2)
    T, E, k = 37, 6, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    s = oracle.build_schedule(idx, E)
    perm = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    perm.append(t * k + j)
    assert list(s.perm) == perm
    assert sorted(s.perm) == list(range(T * k))          # bijection
    assert s.counts.sum() == T * k
    assert list(s.offsets) == [0] + list(np.cumsum([np.sum(idx == e) for e in range(E)]))
    for t in range(T):
        for j in range(k):
            assert s.perm[s.pos[t, j]] == t * k + j       # pos inverts perm
    for e in range(E):                                    # increasing token order inside a segment
        seg = s.perm[s.offsets[e]:s.offsets[e + 1]]
        assert np.all(np.diff(seg // k) > 0)
    assert list(s.padded_offsets) == [0] + list(np.cumsum([-(-c // 32) * 32 for c in s.counts]))


def test_schedule_k_equals_E_selects_all():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((11, 5))
    idx = oracle.select_topk(L, 5)
    assert all(sorted(r) == list(range(5)) for r in idx)
    s = oracle.build_schedule(idx, 5)
    assert np.all(s.counts == 11)


# ---------------------------------------------------------------- experts and combine


def test_combine_identity_experts_returns_x():
    cfg, inp, _ = _tiny(T=32, E=5, k=3, score="sigmoid")
    x = inp.x.astype(np.float64)
    L = oracle.router_logits(x, inp.w_r)
    idx = oracle.select_topk(L, 3)
    w = oracle.routing_weights(L, idx, "sigmoid")
    s = oracle.build_schedule(idx, 5)
    Yrows = x[s.perm // 3]                     # every expert returns its input row
    y = oracle.combine(Yrows, w, s.pos)
    assert np.max(np.abs(y - x)) <= 1e-15 * np.max(np.abs(x)) * 4


def _perm_matrix(n, shift):
    P = np.zeros((n, n))
    P[np.arange(n), (np.arange(n) * 3 + shift) % n] = 1.0  # row i picks column (3i+shift) mod n
    return P


@pytest.mark.parametrize("quant", [False, True])
def test_permutation_experts_closed_form(quant):
    """Experts whose gate, up and down matrices are permutations have a closed-form output.

    With W1 gate = Pg, W1 up = 2 Pu, W2 = Pd (d == I): G = X Pg^T, U = 2 X Pu^T,
    h = silu(G) U, Y = Q(h) Pd^T, so y[t] = sum_j w_j Y_j[t].  A swapped gate/up,
    a transposed operand or a wrong row order changes the result.
    """
    T, d, E, k = 8, 64, 3, 2
    cfg = moe_inputs.LayerConfig("p", T=T, d=d, E=E, k=k, inter=d, score="softmax", seed=5)
    inp = moe_inputs.layer_inputs(cfg)
    x = inp.x.astype(np.float64)
    mats = {}
    for e in range(E):
        Pg, Pu, Pd = _perm_matrix(d, e), _perm_matrix(d, e + 7), _perm_matrix(d, 2 * e + 1)
        mats[e] = (np.concatenate([Pg, 2 * Pu]), Pd)
    fw = oracle.layer_forward(x, inp.w_r, lambda e: mats[e], k, "softmax", quant=quant)
    if quant:
        xq, xs = oracle.quantize(x, axis=1)
        X = oracle.dequantize(xq, xs, axis=1)
    else:
        X = x
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = fw.idx[t, j]
            Pg, Pu2 = mats[e][0][:d], mats[e][0][d:]
            Pd = mats[e][1]
            g = np.array([X[t, np.argmax(Pg[i])] for i in range(d)])       # (X Pg^T)_i = X[p(i)]
            u = np.array([2 * X[t, np.argmax(Pu2[i])] for i in range(d)])
            h = g / (1 + np.exp(-g)) * u
            if quant:
                hq, hs = oracle.quantize(h.astype(np.float32).astype(np.float64)[None], axis=1)
                h = oracle.dequantize(hq, hs, axis=1)[0]
            Yv = np.array([h[np.argmax(Pd[n])] for n in range(d)])
            y[t] += fw.w[t, j] * Yv
    assert np.allclose(fw.y, y, rtol=1e-13, atol=1e-13)


def test_shared_expert_adds_weight_one_row():
    cfg, inp, ws = _tiny(T=8, E=4, k=2, n_shared=1, score="sigmoid")
    ex = oracle.oracle_experts([w[0] for w in ws], [w[1] for w in ws])
    fw1 = oracle.layer_forward(inp.x, inp.w_r, ex, 2, "sigmoid", n_shared=1)
    fw0 = oracle.layer_forward(inp.x, inp.w_r, ex, 2, "sigmoid", n_shared=0)
    shared = oracle.expert_forward(fw0.X, *ex(4)).Y
    assert np.allclose(fw1.y, fw0.y + shared, rtol=1e-13, atol=1e-13)


def test_token_requant_blocks_start_at_segment():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((40, 8)).astype(np.float32).astype(np.float64)
    r = oracle.token_requant(a)
    q0, s0 = oracle.quantize(a[:32], axis=0)
    assert np.array_equal(r[:32], oracle.dequantize(q0, s0, axis=0))
    tail = np.zeros((32, 8))
    tail[:8] = a[32:]
    q1, s1 = oracle.quantize(tail, axis=0)
    assert np.array_equal(r[32:], oracle.dequantize(q1, s1, axis=0)[:8])


# ---------------------------------------------------------------- backward by finite differences


@pytest.mark.parametrize("score,n_shared", [("softmax", 0), ("sigmoid", 0), ("sigmoid", 1)])
def test_backward_matches_finite_differences(score, n_shared):
    cfg, inp, ws = _tiny(T=6, d=32, E=4, k=2, I=32, score=score, seed=21, n_shared=n_shared)
    x = inp.x.astype(np.float64)
    w_r = inp.w_r.astype(np.float64) * 4.0  # spread logits: no near-ties under perturbation
    dy = inp.dy.astype(np.float64)
    W1 = [w[0].astype(np.float64) for w in ws]
    W2 = [w[1].astype(np.float64) for w in ws]

    def loss(x_, w_r_, W1_, W2_):
        ex = lambda e: (W1_[e], W2_[e])
        fw = oracle.layer_forward(x_, w_r_, ex, cfg.k, score, n_shared=n_shared, quant=False)
        return float(np.sum(fw.y * dy))

    ex = lambda e: (W1[e], W2[e])
    fw = oracle.layer_forward(x, w_r, ex, cfg.k, score, n_shared=n_shared, quant=False)
    bw = oracle.layer_backward(fw, dy, x, w_r, ex, score, quant=False)
    rng = np.random.default_rng(0)
    h = 1e-6

    def fd(arr, i, fn):
        old = arr[i]
        arr[i] = old + h
        lp = fn()
        arr[i] = old - h
        lm = fn()
        arr[i] = old
        return (lp - lm) / (2 * h)

    for _ in range(12):
        i = (rng.integers(cfg.T), rng.integers(cfg.d))
        g = fd(x, i, lambda: loss(x, w_r, W1, W2))
        assert abs(g - bw.dx[i]) <= 1e-6 * (1 + abs(g))
        i = (rng.integers(cfg.E), rng.integers(cfg.d))
        g = fd(w_r, i, lambda: loss(x, w_r, W1, W2))
        assert abs(g - bw.dw_r[i]) <= 1e-6 * (1 + abs(g))
        e = int(rng.integers(cfg.E + n_shared))
        i = (rng.integers(2 * cfg.inter), rng.integers(cfg.d))
        g = fd(W1[e], i, lambda: loss(x, w_r, W1, W2))
        assert abs(g - bw.dW1[e][i]) <= 1e-6 * (1 + abs(g))
        i = (rng.integers(cfg.d), rng.integers(cfg.inter))
        g = fd(W2[e], i, lambda: loss(x, w_r, W1, W2))
        assert abs(g - bw.dW2[e][i]) <= 1e-6 * (1 + abs(g))


def test_quantized_backward_shapes_and_zero_experts():
    cfg, inp, ws = _tiny(T=4, d=64, E=8, k=1, I=32, score="softmax", seed=3)
    ex = oracle.oracle_experts([w[0] for w in ws], [w[1] for w in ws])
    fw = oracle.layer_forward(inp.x, inp.w_r, ex, 1, "softmax")
    bw = oracle.layer_backward(fw, inp.dy, inp.x, inp.w_r, ex, "softmax")
    empty = [e for e in range(8) if fw.sched.counts[e] == 0]
    assert empty, "with 4 tokens and 8 experts some expert is empty"
    for e in empty:
        assert not np.any(bw.dW1[e]) and not np.any(bw.dW2[e])
    assert bw.dx.shape == (4, 64) and bw.dw_r.shape == (8, 64)
    # k = 1 softmax: the weight is constant 1, so the router gets no gradient
    assert np.all(bw.dL == 0) and np.all(bw.dw_r == 0)
