"""Full-size parity at the DeepSeek-V3 shape, in the launch configuration bench.py times.

T=8192, d=7168, 256 experts, top-8 sigmoid-normalised routing, I=2048, seed 4 (forward +
backward).  The oracle cannot run the whole layer in a test's time, so it checks what it can
compute piece by piece on the same seeded inputs:

* routing of every token (top-k on float32 logits) and the whole schedule, bit-exact;
* x and dy quantisation, bit-exact;
* six experts (least, median and most loaded, three seeded others) through every stage on the
  GPU's own intermediates (stages.py): quantised weights, W1t / W2t and the token-axis operands
  bit-exact, H and [dG dU] codes exact outside the float32 slack of a rounding boundary, G, U, Y
  slots, dX slots, dW1 and dW2 within 1e-2 RMS;
* dw, dL of every token and the whole dW_router within 1e-2 RMS;
* a sampled token through the combine and the dx reduction within 1e-2 RMS, and against the
  oracle's own end-to-end result within 1e-2 RMS + the envelope of code flips.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
from oracle import envelope
from oracle.layer import _qdq
import stages
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


@pytest.fixture(scope="module")
def view(run):
    cfg, inp, layer, experts = run
    return stages.LayerView(cfg, inp, layer)


def _picks(v, n_random=3):
    """Least-loaded, median-load and most-loaded expert, and a few others (seeded)."""
    counts = v.counts[:v.cfg.E]
    order = np.argsort(counts, kind="stable")
    rng = np.random.default_rng(4)
    picks = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    picks += [int(e) for e in rng.choice(np.setdiff1d(np.arange(v.cfg.E), picks), n_random, replace=False)]
    return picks


def test_sampled_experts_every_stage(run, view):
    """Every stage of six experts on the GPU's own intermediates (stages.py): W1t / W2t, the
    token-axis operands bit-exact; H and [dG dU] codes exact outside the float32 slack; G, U,
    Y slots, dX slots, dW1, dW2 within 1e-2 RMS."""
    cfg, inp, layer, experts = run
    st = stages.StageStats()
    for e in _picks(view):
        log(f"dsv3: expert {e} ({int(view.counts[e])} rows): forward stages")
        w1, w2 = moe_inputs.expert_weights(cfg, e)
        W1, W2, _ = stages.check_expert_forward(view, e, w1, w2, st)
        log(f"dsv3: expert {e}: backward stages")
        stages.check_expert_backward(view, e, W1, W2, st)
    st.report("dsv3")


def test_router_backward_every_token(run, view):
    """dw, dL on every token and the whole dW_router, from the GPU's Y slots, logits and weights."""
    cfg, inp, layer, experts = run
    st = stages.StageStats()
    dL = stages.check_router_backward(view, st)
    dLfull = np.zeros((cfg.T, cfg.E))
    np.put_along_axis(dLfull, view.idx.astype(np.int64), dL, axis=1)
    st.err("dW_router", to_np(layer.dw_r), dLfull.T @ inp.x.astype(np.float64))
    st.report("dsv3")


@pytest.mark.parametrize("t", [4321])
def test_sampled_token_end_to_end(run, view, t):
    """One token through every stage (its k experts): the combine of its Y slots into y, and dx
    from its dX slot rows (oracle dgrad of the GPU's [dG dU]) plus the router term, both within
    1e-2 RMS; then the token against the oracle's own end-to-end result within 1e-2 RMS plus the
    admissible envelope of the code flips (a secondary check)."""
    cfg, inp, layer, experts = run
    st = stages.StageStats()
    ys = to_np(layer.saved_tensor("yslot")[t]).astype(np.float64)
    st.err(f"y[{t}]", to_np(layer.y32[t]), view.w[t] @ ys[:cfg.k])
    # dX slot rows of the token from the GPU's [dG dU] rows
    rows = view.pos[t]
    dguq = to_np(layer.workspace_tensor("dguq")[rows])
    dgus = to_np(layer.workspace_tensor("dgus")[rows])
    DGU = oracle.dequantize(dguq, dgus, axis=1)
    dX = np.zeros((cfg.k, cfg.d))
    for j, e in enumerate(view.idx[t]):
        W1t = _qdq(experts(int(e))[0], 0, True)[2]
        dX[j] = DGU[j] @ W1t
    st.err(f"dX slots[{t}]", to_np(layer.workspace_tensor("dxslot")[t]), dX)
    dL = stages.check_router_backward(view, st, tokens=[t])[0]
    wr = inp.w_r.astype(np.float64)
    dx = dX.sum(axis=0) + dL @ wr[view.idx[t]]
    st.err(f"dx[{t}]", to_np(layer.dx32[t]), dx)
    st.report("dsv3")
    # secondary: the oracle's own end-to-end result, within 1e-2 RMS + the envelope of code flips
    x = inp.x[t:t + 1].astype(np.float64)
    dy = inp.dy[t:t + 1].astype(np.float64)
    log(f"dsv3: token {t}: oracle forward / backward / envelopes")
    fw = oracle.layer_forward(x, inp.w_r, experts, cfg.k, cfg.score)
    bw = oracle.layer_backward(fw, dy, x, inp.w_r, experts, cfg.score, expert_subset=sorted(fw.experts))
    fenv = envelope.forward_envelope(fw, experts, EPS)
    benv = envelope.backward_envelope(fw, bw, fenv, dy, x, inp.w_r, experts, cfg.score)
    assert np.array_equal(to_np(layer.saved_tensor("idx")[t]), fw.idx[0])
    _check(f"y[{t}] end to end", to_np(layer.y32[t:t + 1]), fw.y, fenv.By)
    _check(f"dx[{t}] end to end", to_np(layer.dx32[t:t + 1]), bw.dx, benv.Bdx)


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


def test_ring_dispatch_bitwise_at_full_size(run):
    """The ring dispatch at its default capacity (16,384 rows: 64 slots, rounds of 32 chunks) and
    producer count, forward (x rows) and backward (dY rows), on the same experts: every output and
    gradient bit for bit those of the direct pull."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import MoeLayer
    cfg, inp, layer, experts = run
    ring = MoeLayer.from_config(cfg, with_backward=True, flags=moe.MOE_F_RING_DISPATCH)
    ring.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits)
    for a, b in ((ring.w1q, layer.w1q), (ring.w1s, layer.w1s), (ring.w2q, layer.w2q), (ring.w2s, layer.w2s)):
        a.copy_(b)
    log("dsv3: forward + backward through the ring")
    ring.forward()
    ring.backward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(ring.workspace) == 0
    names = ("y", "y32", "dx", "dx32", "dw_r", "dw1", "dw2")
    for name in names:
        assert torch.equal(getattr(ring, name), getattr(layer, name)), name
    for name in ("g", "u", "hq", "hs", "yslot"):
        assert torch.equal(ring.saved_tensor(name), layer.saved_tensor(name)), name
    del ring
    torch.cuda.empty_cache()


def test_bf16_weight_gradients_at_full_size(run):
    """MOE_F_DW_BF16 at the DSV3 shape: dW1 and dW2 in bf16 are the default float32 gradients
    rounded to nearest, ties to even, bit for bit (22.6 GB written instead of 45.2 GB)."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import MoeLayer
    cfg, inp, layer, experts = run
    b16 = MoeLayer.from_config(cfg, with_backward=True, flags=moe.MOE_F_DW_BF16)
    b16.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits)
    for a, b in ((b16.w1q, layer.w1q), (b16.w1s, layer.w1s), (b16.w2q, layer.w2q), (b16.w2s, layer.w2s)):
        a.copy_(b)
    log("dsv3: forward + backward with bf16 weight gradients")
    b16.forward()
    b16.backward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(b16.workspace) == 0
    for name, a, b in (("dW1", layer.dw1, b16.dw1), ("dW2", layer.dw2, b16.dw2)):
        for e0 in range(0, a.shape[0], 32):  # in slices: the rounded copy of a whole fp32 dW1 is 15 GB
            assert torch.equal(a[e0:e0 + 32].to(torch.bfloat16).view(torch.int16),
                               b[e0:e0 + 32].view(torch.int16)), (name, e0)
    assert torch.equal(layer.dx32, b16.dx32)
    del b16
    torch.cuda.empty_cache()

