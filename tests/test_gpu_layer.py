"""The layer on the GPU against the oracle on the same seeded inputs.

Bit-exact: top-k selection, schedule (counts, offsets, permutation, inverse), quantised x.
Gate/up results: within the accumulation model |G_gpu - G| <= EPS * sum|a b|.
H codes: equal to the oracle's wherever the oracle's code is unique, admissible elsewhere
(oracle.envelope: a float32 accumulation may legitimately land on the neighbouring code).
Float outputs (y, Y slots, dx, dW_router, dW1, dW2, on the float32 copies):
max |err| <= 1e-2 x RMS of the oracle tensor + the oracle's admissible envelope; the bf16
outputs equal the float32 copies rounded to nearest even.  Bitwise identical across runs.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
from oracle import envelope
from helpers import gpu_layer, log, oracle_layer, rel_err, rms, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2
EPS = 2.0 ** -15  # accumulation model of the matrix-core GEMMs (checked on G and U)

MID = moe_inputs.LayerConfig("mid", T=512, d=512, E=16, k=4, inter=256, score="softmax", seed=7)
MID_SIG = moe_inputs.LayerConfig("mid_sig_shared", T=384, d=256, E=24, k=6, inter=384, score="sigmoid", seed=8,
                                 n_shared=1, zipf_s=1.1, zipf_lam=0.5)
# Edge cases: a ragged token count (not a multiple of any tile or block) with 12 experts; a
# strongly skewed router that leaves 8 of 16 experts without rows and one with a single row;
# k = E (every expert sees every token, T ragged); k = 1 with a shared expert and d = 384 (an odd
# number of K stages); the routing limits.
RAGGED = moe_inputs.LayerConfig("ragged", T=200, d=256, E=12, k=3, inter=128, score="softmax", seed=9)
EMPTY = moe_inputs.LayerConfig("empty_experts", T=72, d=128, E=16, k=2, inter=128, score="sigmoid", seed=10,
                               zipf_s=1.1, zipf_lam=2.0)
K_EQ_E = moe_inputs.LayerConfig("k_eq_e", T=65, d=128, E=4, k=4, inter=256, score="softmax", seed=11)
K1_SHARED = moe_inputs.LayerConfig("k1_shared", T=130, d=384, E=6, k=1, inter=128, score="sigmoid", seed=12,
                                   n_shared=1)
# the API's routing limits: 512 experts, top-16 (most experts see a few rows, many none)
MAX_ROUTE = moe_inputs.LayerConfig("max_route", T=70, d=128, E=512, k=16, inter=128, score="softmax", seed=13)
CASES = [moe_inputs.CONFIGS["tiny"], MID, MID_SIG, RAGGED, EMPTY, K_EQ_E, K1_SHARED, MAX_ROUTE]


def _bf16_rne(a32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


@pytest.fixture(scope="module", params=CASES, ids=lambda c: c.name)
def pair(request):
    cfg = request.param.with_(backward=True)
    log(f"case {cfg.name}: oracle")
    inp, ws, ex, fw, bw = oracle_layer(cfg, True)
    log(f"case {cfg.name}: gpu")
    layer = gpu_layer(cfg, True, inp=inp, ws=ws)
    return cfg, inp, fw, bw, layer


def test_schedule_bit_exact(pair):
    cfg, inp, fw, bw, layer = pair
    if cfg.name == "empty_experts":  # the case it stands for
        assert np.sum(fw.sched.counts == 0) >= 4
    if cfg.name == "k_eq_e":
        assert np.all(fw.sched.counts == cfg.T)
    idx = to_np(layer.saved_tensor("idx"))
    L = to_np(layer.saved_tensor("logits")).astype(np.float64)
    # logits: float32 accumulation of exact bf16 products
    bound = 1e-5 * (np.abs(inp.x.astype(np.float64)) @ np.abs(inp.w_r.astype(np.float64)).T) + 1e-30
    assert np.all(np.abs(L - fw.L) <= bound)
    assert np.array_equal(idx, fw.idx)
    assert np.array_equal(to_np(layer.saved_tensor("perm")), fw.sched.perm)
    assert np.array_equal(to_np(layer.saved_tensor("pos")), fw.sched.pos)
    NX = cfg.E + cfg.n_shared
    counts = np.concatenate([fw.sched.counts, np.full(cfg.n_shared, cfg.T)])
    assert np.array_equal(to_np(layer.saved_tensor("counts")), counts)
    offs = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(to_np(layer.saved_tensor("offsets")), offs)
    poffs = np.concatenate([[0], np.cumsum(-(-counts // 32) * 32)])
    assert np.array_equal(to_np(layer.saved_tensor("poffsets")), poffs)
    assert np.array_equal(to_np(layer.saved_tensor("poffsets"))[: cfg.E + 1], fw.sched.padded_offsets)
    w = to_np(layer.saved_tensor("w"))
    assert np.max(np.abs(w - fw.w)) <= 1e-5
    assert layer.saved_tensor("counts").shape[0] == NX


def test_quantised_x_bit_exact(pair):
    cfg, inp, fw, bw, layer = pair
    assert np.array_equal(to_np(layer.saved_tensor("xq")), fw.xq)
    assert np.array_equal(to_np(layer.saved_tensor("xs")), fw.xs)


def _expert_rows(fw, name):
    parts = [getattr(fw.experts[e], name) for e in sorted(fw.experts)]
    return np.concatenate(parts, axis=0)


def _rows(d, fw):
    return np.concatenate([d[e] for e in sorted(fw.experts)], axis=0)


@pytest.fixture(scope="module")
def env(pair):
    cfg, inp, fw, bw, layer = pair
    _, ws, ex, _, _ = oracle_layer(cfg, True)
    fenv = envelope.forward_envelope(fw, ex, EPS)
    benv = envelope.backward_envelope(fw, bw, fenv, inp.dy, inp.x, inp.w_r, ex, cfg.score)
    return fenv, benv


def _check(name, got, ref, bound):
    """max |got - ref| <= TOL * RMS(ref) + bound (elementwise); log how much of the envelope was used."""
    got = np.asarray(got, dtype=np.float64)
    r = rms(ref)
    err = np.abs(got - ref)
    beyond = err > TOL * r
    if r > 0:
        log(f"  {name}: max|err|/rms {err.max() / r:.3e}; elements beyond {TOL:g} rms: {int(beyond.sum())} "
            f"({beyond.mean():.2e}); envelope max {bound.max() / r:.2e} mean {bound.mean() / r:.2e} rms")
    else:  # an exactly zero reference (e.g. the router gradient with k = 1 and normalised weights)
        log(f"  {name}: reference is zero; max|err| {err.max():.3e}, envelope max {bound.max():.3e}")
    assert np.all(err <= TOL * r + bound), name


def test_gate_up_within_accumulation_model(pair, env):
    cfg, inp, fw, bw, layer = pair
    fenv, _ = env
    G = to_np(layer.saved_tensor("g")).astype(np.float64)
    U = to_np(layer.saved_tensor("u")).astype(np.float64)
    eG, eU = _rows(fenv.eG, fw), _rows(fenv.eU, fw)
    dG = np.abs(G - _expert_rows(fw, "G"))
    dU = np.abs(U - _expert_rows(fw, "U"))
    log(f"{cfg.name}: |G err| / model max {np.max(dG / eG):.3f}, |U err| / model max {np.max(dU / eU):.3f}")
    assert np.all(dG <= eG) and np.all(dU <= eU)


def test_h_codes_admissible(pair, env):
    cfg, inp, fw, bw, layer = pair
    fenv, _ = env
    hq = to_np(layer.saved_tensor("hq"))
    hs = to_np(layer.saved_tensor("hs"))
    H = oracle.dequantize(hq, hs, axis=1)
    lo, hi = _rows(fenv.H_lo, fw), _rows(fenv.H_hi, fw)
    unique = lo == hi
    Href = _expert_rows(fw, "H")
    log(f"{cfg.name}: H ambiguous fraction {1 - unique.mean():.3e}; codes differing {np.mean(H != Href):.3e}")
    assert np.all(H[unique] == Href[unique])
    assert np.all((H >= lo) & (H <= hi))


def test_forward_output(pair, env):
    cfg, inp, fw, bw, layer = pair
    fenv, _ = env
    import torch
    log(f"{cfg.name}: forward")
    _check("y", to_np(layer.y32), fw.y, fenv.By)
    assert np.array_equal(to_np(layer.y.view(torch.int16)), _bf16_rne(to_np(layer.y32)))
    ys = to_np(layer.saved_tensor("yslot"))
    _check("Y slots", ys[:, : cfg.k].reshape(-1, cfg.d), fw.Yrows[fw.sched.pos.reshape(-1)],
           fenv.BY[fw.sched.pos.reshape(-1)])


def test_backward_outputs(pair, env):
    cfg, inp, fw, bw, layer = pair
    fenv, benv = env
    import torch
    NX = cfg.E + cfg.n_shared
    log(f"{cfg.name}: backward")
    _check("dx", to_np(layer.dx32), bw.dx, benv.Bdx)
    _check("dW_router", to_np(layer.dw_r), bw.dw_r, benv.Bdw_r)
    zero = {e: np.zeros_like(bw.dW1[e]) for e in range(NX)}
    _check("dW1", to_np(layer.dw1), np.stack([bw.dW1[e] for e in range(NX)]),
           np.stack([benv.BdW1.get(e, zero[e]) for e in range(NX)]))
    zero2 = {e: np.zeros_like(bw.dW2[e]) for e in range(NX)}
    _check("dW2", to_np(layer.dw2), np.stack([bw.dW2[e] for e in range(NX)]),
           np.stack([benv.BdW2.get(e, zero2[e]) for e in range(NX)]))
    assert np.array_equal(to_np(layer.dx.view(torch.int16)), _bf16_rne(to_np(layer.dx32)))


def test_bitwise_reproducible(pair):
    cfg, inp, fw, bw, layer = pair
    import torch
    ref = [t.clone() for t in (layer.y32, layer.y, layer.dx32, layer.dw_r, layer.dw1, layer.dw2)]
    for _ in range(10):
        layer.forward()
        layer.backward()
        torch.cuda.synchronize()
        for r, t in zip(ref, (layer.y32, layer.y, layer.dx32, layer.dw_r, layer.dw1, layer.dw2)):
            assert torch.equal(r, t)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_identity_experts_return_x(cfg):
    """Identity experts with unit-sum combine weights (plus weight-1 shared experts): the layer
    returns (1 + n_shared) x, bit for bit in bf16 (a sum of k weights is 1 within a few float32
    ulps, far inside half a bf16 ulp), on the GPU's own routing."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import MoeLayer
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    layer = MoeLayer.from_config(cfg, with_backward=True, flags=moe.MOE_F_IDENTITY_EXPERTS)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits)
    layer.load_experts(moe_inputs.iter_expert_weights(cfg))
    layer.forward()
    torch.cuda.synchronize()
    x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).float()
    ref = (1 + cfg.n_shared) * x  # exact
    assert torch.equal(layer.y.cpu().view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))
    y32 = layer.y32.cpu()
    assert torch.all((y32 - ref).abs() <= 2.0 ** -20 * ref.abs())
    w = to_np(layer.saved_tensor("w"))
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 4 * 2.0 ** -24 * cfg.k
    with pytest.raises(moe.MoeError):
        layer.backward()


def test_serial_and_concurrent_backward_identical(pair):
    """The backward's second-stream schedule (default) and the launch-order schedule
    (MOE_F_SERIAL_BWD) produce bitwise identical gradients."""
    cfg, inp, fw, bw, layer = pair
    import torch
    import mixture_experts_layer_schedule_amd as moe
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (layer.dx32, layer.dw1, layer.dw2, layer.dw_r)]
    layer.cfg.flags |= moe.MOE_F_SERIAL_BWD
    try:
        for t in (layer.dx32, layer.dw1, layer.dw2, layer.dw_r):
            t.zero_()
        layer.backward()
        torch.cuda.synchronize()
    finally:
        layer.cfg.flags &= ~moe.MOE_F_SERIAL_BWD
    for name, a, b in zip(("dx", "dW1", "dW2", "dW_r"), ref, (layer.dx32, layer.dw1, layer.dw2, layer.dw_r)):
        assert torch.equal(a, b), name
