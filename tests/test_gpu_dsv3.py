"""Full-size parity at the DeepSeek-V3 shape, in the launch configuration bench.py times.

T=8192, d=7168, 256 experts, top-8 sigmoid-normalised routing, I=2048, seed 4 (forward +
backward).  The oracle cannot run the whole layer in a test's time, so it checks what it can
compute piece by piece on the same seeded inputs:

* routing of every token (top-k on float32 logits) and the whole schedule, bit-exact;
* x quantisation, bit-exact;
* two experts (median and maximum load) end to end: G/U within the accumulation model, H codes
  unique-or-admissible, their Y rows, dW1 and dW2 within 1e-2 RMS + envelope;
* a sampled token end to end (all its experts): y and dx within 1e-2 RMS + envelope.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
from oracle import envelope
from oracle.layer import _qdq
from helpers import log, rms, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2
EPS = 2.0 ** -15
CFG = moe_inputs.CONFIGS["dsv3_fwd_bwd"]


@pytest.fixture(scope="module")
def run():
    import torch
    from mixture_experts_layer_schedule_amd import MoeLayer
    import mixture_experts_layer_schedule_amd as moe

    cfg = CFG
    log(f"dsv3: inputs and {cfg.E} experts")
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    layer = MoeLayer.from_config(cfg, with_backward=True)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits)
    layer.load_experts(moe_inputs.iter_expert_weights(cfg, threads=16))
    log("dsv3: forward + backward")
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(layer.workspace) == 0
    cache = {}

    def experts(e):
        if e not in cache:
            log(f"dsv3: oracle weights of expert {e}")
            w1, w2 = moe_inputs.expert_weights(cfg, e)
            cache[e] = (_qdq(w1, 1, True)[2], _qdq(w2, 1, True)[2])
        return cache[e]

    return cfg, inp, layer, experts


def test_routing_and_schedule(run):
    cfg, inp, layer, experts = run
    x = inp.x.astype(np.float64)
    L = oracle.router_logits(x, inp.w_r)
    idx = oracle.select_topk(L, cfg.k)
    gidx = to_np(layer.saved_tensor("idx"))
    diff = np.where(np.any(gidx != idx, axis=1))[0]
    log(f"dsv3: tokens whose selection differs from the oracle: {len(diff)}")
    gL = to_np(layer.saved_tensor("logits")).astype(np.float64)
    bound = 1e-5 * (np.abs(x) @ np.abs(inp.w_r.astype(np.float64)).T)
    assert np.all(np.abs(gL - L) <= bound)
    # A differing selection (or order of the selected experts) must be a near-tie that float32
    # logits cannot order: at the first rank where the two lists differ, both experts were the
    # best of the same remaining set, so their exact logits are within the two logits' bounds.
    for t in diff:
        p = int(np.argmax(gidx[t] != idx[t]))
        assert abs(L[t, gidx[t, p]] - L[t, idx[t, p]]) <= 2 * bound[t].max(), t
    if len(diff) == 0:
        sched = oracle.build_schedule(idx, cfg.E)
        assert np.array_equal(to_np(layer.saved_tensor("perm")), sched.perm)
        assert np.array_equal(to_np(layer.saved_tensor("pos")), sched.pos)
        assert np.array_equal(to_np(layer.saved_tensor("counts")), sched.counts)
    # schedule invariants on the GPU's own selection
    perm = to_np(layer.saved_tensor("perm"))
    assert np.array_equal(np.sort(perm), np.arange(cfg.T * cfg.k))
    assert np.array_equal(perm, oracle.build_schedule(gidx, cfg.E).perm)
    w = oracle.routing_weights(L, idx, cfg.score)
    assert np.max(np.abs(to_np(layer.saved_tensor("w")) - w)) <= 1e-5


def test_x_quantised_bit_exact(run):
    cfg, inp, layer, experts = run
    xq, xs = oracle.quantize(inp.x.astype(np.float64), axis=1)
    assert np.array_equal(to_np(layer.saved_tensor("xq")), xq)
    assert np.array_equal(to_np(layer.saved_tensor("xs")), xs)


def _check(name, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    r = rms(ref)
    err = np.abs(got - ref)
    log(f"  {name}: max|err|/rms {err.max() / r:.3e}; beyond {TOL:g} rms: {int((err > TOL * r).sum())}; "
        f"envelope max {bound.max() / r:.2e} mean {bound.mean() / r:.2e} rms")
    assert np.all(err <= TOL * r + bound), name


def test_sampled_experts_end_to_end(run):
    cfg, inp, layer, experts = run
    counts = to_np(layer.saved_tensor("counts"))
    offs = to_np(layer.saved_tensor("offsets"))
    perm = to_np(layer.saved_tensor("perm"))
    wflat = oracle.routing_weights(oracle.router_logits(inp.x, inp.w_r), to_np(layer.saved_tensor("idx")),
                                   cfg.score).reshape(-1)
    order = np.argsort(counts)
    picks = [int(order[len(order) // 2]), int(order[-1])]
    xq, xs = oracle.quantize(inp.x.astype(np.float64), axis=1)
    X = oracle.dequantize(xq, xs, axis=1)
    dyq, dys = oracle.quantize(inp.dy.astype(np.float64), axis=1)
    DY = oracle.dequantize(dyq, dys, axis=1)
    G = layer.saved_tensor("g")
    U = layer.saved_tensor("u")
    for e in picks:
        lo, hi = int(offs[e]), int(offs[e + 1])
        toks = perm[lo:hi] // cfg.k
        wrow = wflat[perm[lo:hi]]
        W1, W2 = experts(e)
        log(f"dsv3: expert {e} with {hi - lo} rows")
        fe = oracle.expert_forward(X[toks], W1, W2)
        eG, eU, Hlo, Hhi, devH, BY = envelope.expert_forward_envelope(fe, X[toks], W1, W2, EPS)
        g = to_np(G[lo:hi]).astype(np.float64)
        u = to_np(U[lo:hi]).astype(np.float64)
        log(f"  G err / model max {np.max(np.abs(g - fe.G) / eG):.3f}")
        assert np.all(np.abs(g - fe.G) <= eG) and np.all(np.abs(u - fe.U) <= eU)
        H = oracle.dequantize(to_np(layer.saved_tensor("hq")[lo:hi]), to_np(layer.saved_tensor("hs")[lo:hi]), axis=1)
        uniq = Hlo == Hhi
        assert np.all(H[uniq] == fe.H[uniq]) and np.all((H >= Hlo) & (H <= Hhi))
        ys = layer.saved_tensor("yslot").view(-1, cfg.d)
        slots = (perm[lo:hi] // cfg.k) * cfg.k + perm[lo:hi] % cfg.k
        _check(f"Y rows of expert {e}", to_np(ys[slots]), fe.Y, BY)
        W2t = _qdq(W2, 0, True)[2]
        W1t = _qdq(W1, 0, True)[2]
        be = oracle.expert_backward(fe, X[toks], DY[toks], wrow, W1t, W2t)
        _, _, _, bdw1, bdw2 = envelope.expert_backward_envelope(fe, be, X[toks], DY[toks], wrow, W1, W2, eG, eU,
                                                                devH, EPS)
        _check(f"dW1[{e}]", to_np(layer.dw1[e]), be.dW1, bdw1)
        _check(f"dW2[{e}]", to_np(layer.dw2[e]), be.dW2, bdw2)


@pytest.mark.parametrize("t", [4321])
def test_sampled_token_end_to_end(run, t):
    cfg, inp, layer, experts = run
    x = inp.x[t:t + 1].astype(np.float64)
    dy = inp.dy[t:t + 1].astype(np.float64)
    log(f"dsv3: token {t}: oracle forward")
    fw = oracle.layer_forward(x, inp.w_r, experts, cfg.k, cfg.score)
    log(f"dsv3: token {t}, experts {list(fw.idx[0])}: oracle backward")
    bw = oracle.layer_backward(fw, dy, x, inp.w_r, experts, cfg.score, expert_subset=sorted(fw.experts))
    log(f"dsv3: token {t}: envelopes")
    fenv = envelope.forward_envelope(fw, experts, EPS)
    benv = envelope.backward_envelope(fw, bw, fenv, dy, x, inp.w_r, experts, cfg.score)
    assert np.array_equal(to_np(layer.saved_tensor("idx")[t]), fw.idx[0])
    _check(f"y[{t}]", to_np(layer.y32[t:t + 1]), fw.y, fenv.By)
    _check(f"dx[{t}]", to_np(layer.dx32[t:t + 1]), bw.dx, benv.Bdx)


def test_bitwise_run_to_run(run):
    """A second forward + backward of the same inputs reproduces every output bit for bit (fixed
    summation orders, no atomics), in the default two-stream backward schedule."""
    import torch
    cfg, inp, layer, experts = run
    outs = lambda: (layer.y, layer.y32, layer.dx, layer.dx32, layer.dw_r, layer.dw1, layer.dw2)  # noqa: E731
    ref = [t.clone() for t in outs()]
    log("dsv3: second forward + backward")
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    for name, r, t in zip(("y", "y32", "dx", "dx32", "dw_r", "dw1", "dw2"), ref, outs()):
        assert torch.equal(r, t), name
    del ref
    torch.cuda.empty_cache()
