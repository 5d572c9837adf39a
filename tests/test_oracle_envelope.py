"""Pin of the admissible envelope: perturbed accumulations stay inside it.

Every accumulated value is pushed to (random) points of its allowed error interval,
the layer's later steps are recomputed from there, and each output must stay inside
the envelope the oracle computed without seeing any perturbation.
"""
import numpy as np

import moe_inputs
import oracle
from oracle import envelope
from oracle.layer import _f32, _qdq, _sigmoid, token_requant


def _setup(score="sigmoid", n_shared=0, seed=31):
    cfg = moe_inputs.LayerConfig("env", T=64, d=128, E=6, k=3, inter=64, score=score, seed=seed,
                                 n_shared=n_shared)
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + n_shared)]
    ex = oracle.oracle_experts([w[0] for w in ws], [w[1] for w in ws])
    fw = oracle.layer_forward(inp.x, inp.w_r, ex, cfg.k, score, n_shared=n_shared)
    bw = oracle.layer_backward(fw, inp.dy, inp.x, inp.w_r, ex, score)
    return cfg, inp, ex, fw, bw


def _push(rng, a, err, scale=1.0):
    """A point of [a - err, a + err]: mostly at the ends, where codes flip."""
    r = rng.choice([-1.0, 1.0], size=a.shape) * np.where(rng.random(a.shape) < 0.7, 1.0, rng.random(a.shape))
    return a + scale * r * err


def test_forward_envelope_contains_perturbed_results():
    eps = 2.0 ** -10  # wide enough that many codes are ambiguous
    cfg, inp, ex, fw, bw = _setup()
    env = envelope.forward_envelope(fw, ex, eps)
    rng = np.random.default_rng(0)
    flips = 0
    for trial in range(6):
        Yrows = fw.Yrows.copy()
        for e, fe in fw.experts.items():
            W1, W2 = ex(e)
            G = _push(rng, fe.G, env.eG[e])
            U = _push(rng, fe.U, env.eU[e])
            h = _f32(G * _sigmoid(G) * U)
            _, _, H = _qdq(h, 1, True)
            flips += int(np.sum(H != fe.H))
            assert np.all(H >= env.H_lo[e]) and np.all(H <= env.H_hi[e])
            lo, hi = fw.sched.offsets[e], fw.sched.offsets[e + 1]
            Yrows[lo:hi] = H @ W2.T
        y = oracle.combine(Yrows, fw.w, fw.sched.pos)
        assert np.all(np.abs(y - fw.y) <= env.By + 1e-12)
    assert flips > 0, "the test must exercise code flips"


def test_backward_envelope_contains_perturbed_results():
    eps = 2.0 ** -10
    cfg, inp, ex, fw, bw = _setup(score="softmax", seed=32)
    fenv = envelope.forward_envelope(fw, ex, eps)
    benv = envelope.backward_envelope(fw, bw, fenv, inp.dy, inp.x, inp.w_r, ex, "softmax")
    rng = np.random.default_rng(1)
    DY = _qdq(inp.dy.astype(np.float64), 1, True)[2]
    flips = 0
    for trial in range(4):
        dXrows = np.zeros_like(fw.Yrows)
        for e, be in bw.experts.items():
            fe = fw.experts[e]
            W1, W2 = ex(e)
            W1t = _qdq(W1, 0, True)[2]
            W2t = _qdq(W2, 0, True)[2]
            lo, hi = fw.sched.offsets[e], fw.sched.offsets[e + 1]
            wrow = fw.w.reshape(-1)[fw.sched.perm[lo:hi]]
            toks = fw.rows_of[e]
            G = _push(rng, fe.G, fenv.eG[e])
            U = _push(rng, fe.U, fenv.eU[e])
            edH = eps * np.abs(wrow)[:, None] * (np.abs(DY[toks]) @ np.abs(W2t))
            dH = _push(rng, be.dH, edH)
            s = _sigmoid(G)
            dGU = _f32(np.concatenate([dH * U * s * (1 + G * (1 - s)), dH * G * s], axis=1))
            _, _, DGU = _qdq(dGU, 1, True)
            flips += int(np.sum(DGU != be.DGU))
            assert np.all(DGU >= benv.GU_lo[e]) and np.all(DGU <= benv.GU_hi[e])
            dXrows[lo:hi] = DGU @ W1t
            dW1 = token_requant(DGU).T @ token_requant(fw.X[toks])
            assert np.all(np.abs(dW1 - bw.dW1[e]) <= benv.BdW1[e] + 1e-12)
            # H moves inside its forward range: dW2 stays inside its bound
            H = fe.H + _push(rng, np.zeros_like(fe.H), fenv.dH[e], 1.0)
            H = np.clip(H, fenv.H_lo[e], fenv.H_hi[e])
            dYw = _f32(_f32(wrow)[:, None] * DY[toks])
            dW2 = token_requant(dYw).T @ token_requant(H)
            assert np.all(np.abs(dW2 - bw.dW2[e]) <= benv.BdW2[e] + 1e-12)
        dx = np.zeros_like(fw.y)
        for j in range(cfg.k):
            dx += dXrows[fw.sched.pos[:, j]]
        dLfull = np.zeros((cfg.T, cfg.E))
        np.put_along_axis(dLfull, fw.idx.astype(np.int64), bw.dL, axis=1)
        dx += dLfull @ inp.w_r.astype(np.float64)
        assert np.all(np.abs(dx - bw.dx) <= benv.Bdx + 1e-12)
    assert flips > 0


def test_envelope_is_zero_without_uncertainty():
    cfg, inp, ex, fw, bw = _setup()
    env = envelope.forward_envelope(fw, ex, 0.0)
    F = envelope.F32_SLACK
    # with exact accumulation only float32 epilogue slack remains: almost every code is unique
    total = sum(v.size for v in env.dH.values())
    ambiguous = sum(int(np.count_nonzero(v)) for v in env.dH.values())
    assert ambiguous <= total * 1e-3 + 2
    assert F < 1e-5


def test_accumulation_model_is_one_value_everywhere():
    """The envelope's default accumulation model is the one the GPU checks use (the GPU tests
    measure the gate/up error against it on every run: up to 2^-15.96 * sum|a b| at K = 256)."""
    import ast
    import os
    import stages
    from oracle import envelope
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    assert envelope.EPS_ACC == stages.EPS == 2.0 ** -15
    for name in ("tests/test_gpu_layer.py", "tests/test_gpu_dsv3.py", "tests/test_gpu_workloads.py"):
        tree = ast.parse(open(os.path.join(root, name)).read())
        eps = [n.value for n in tree.body if isinstance(n, ast.Assign) and
               any(isinstance(t, ast.Name) and t.id == "EPS" for t in n.targets)]
        assert len(eps) == 1 and eval(compile(ast.Expression(eps[0]), name, "eval")) == envelope.EPS_ACC, name
