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

from helpers import CASES, MID_SIG as MID_SIG_CFG  # noqa: E402


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


def test_bf16_weight_gradients_are_the_rounded_float32_ones(pair):
    """MOE_F_DW_BF16 writes dW1 and dW2 in bf16: each element is the float32 gradient of the
    default path rounded to nearest, ties to even, bit for bit; dx and dW_router are unchanged."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    cfg, inp, fw, bw, layer = pair
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    b16 = gpu_layer(cfg, True, inp=inp, ws=ws, flags=moe.MOE_F_DW_BF16)
    assert b16.dw1.dtype == torch.bfloat16 and b16.dw2.dtype == torch.bfloat16
    for name, a, b in (("dW1", layer.dw1, b16.dw1), ("dW2", layer.dw2, b16.dw2)):
        assert torch.equal(a.to(torch.bfloat16).view(torch.int16), b.view(torch.int16)), name
    for name, a, b in (("dx", layer.dx32, b16.dx32), ("dW_r", layer.dw_r, b16.dw_r)):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("rows", [32, 96, 128])
def test_row_tile_height_changes_no_bit(pair, rows):
    """chunk_rows (rows per GEMM row tile, the tuning knob of the direct path) changes the work
    items only: the row-tile table is ceil(count / rows) per expert, and every output, gradient
    and saved or workspace stage result is bitwise that of the default 256-row tiles."""
    cfg, inp, fw, bw, layer = pair
    import torch
    names = ("y", "y32", "dx", "dx32", "dw1", "dw2", "dw_r")
    saved = ("g", "u", "hq", "hs", "yslot")
    work = ("dguq", "dgus", "dxslot")
    layer.cfg.chunk_rows = 0
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    ref = {n: getattr(layer, n).clone() for n in names}
    ref.update({n: layer.saved_tensor(n).clone() for n in saved})
    ref.update({n: layer.workspace_tensor(n).clone() for n in work})
    try:
        layer.cfg.chunk_rows = rows
        for n in names:
            getattr(layer, n).zero_()
        layer.forward()
        layer.backward()
        torch.cuda.synchronize()
        counts = to_np(layer.saved_tensor("counts")).astype(np.int64)
        tiles = np.concatenate([[0], np.cumsum(-(-counts // rows))])
        assert np.array_equal(to_np(layer.saved_tensor("tile_start")), tiles)
        got = {n: getattr(layer, n) for n in names}
        got.update({n: layer.saved_tensor(n) for n in saved})
        got.update({n: layer.workspace_tensor(n) for n in work})
        for n in ref:
            assert torch.equal(ref[n], got[n]), (cfg.name, rows, n)
    finally:
        layer.cfg.chunk_rows = 0


def test_tuner_picks_a_candidate_and_keeps_the_bits():
    """The per-workload tuner times its candidates on a layer and leaves the fastest in its
    configuration; the tuned layer computes the default layer's bits."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import tune
    cfg = moe_inputs.CONFIGS["tiny"].with_(backward=True)
    layer = gpu_layer(cfg, True)
    ref = [t.clone() for t in (layer.y32, layer.dx32, layer.dw1, layer.dw2, layer.dw_r)]
    res = tune.tune(layer, backward=True, steps=1, warmup=1)
    cands = tune.candidates(layer.T, layer.E, layer.k, layer.S, True)
    assert res.best in cands and set(res.ms) == set(cands)
    log("tuner: " + ", ".join(f"{k} {v:.3f}" for k, v in res.table().items()))
    assert layer.cfg.chunk_rows == res.best.chunk_rows
    assert bool(layer.cfg.flags & moe.MOE_F_SERIAL_BWD) == res.best.serial_bwd
    for t in (layer.y32, layer.dx32, layer.dw1, layer.dw2, layer.dw_r):
        t.zero_()
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "dx", "dW1", "dW2", "dW_r"), ref,
                          (layer.y32, layer.dx32, layer.dw1, layer.dw2, layer.dw_r)):
        assert torch.equal(a, b), name


def test_nonfinite_logits_route_to_valid_experts():
    """A token whose router logits are all NaN (a NaN in its x row) still selects k distinct valid
    experts (NaN ranks as -inf, ties to the lower index: experts 0..k-1), the schedule stays a
    bijection, and the device status word reports MOE_DEV_NONFINITE_LOGIT."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    cfg = moe_inputs.CONFIGS["tiny"]
    inp = moe_inputs.layer_inputs(cfg)
    x = inp.x_bits.copy()
    x[5, 7] = 0x7FC0   # a bf16 NaN: every logit of token 5 is NaN
    x[9, 3] = 0x7F80   # +inf: token 9's logits are +-inf or NaN
    layer = gpu_layer(cfg, False, inp=moe_inputs.LayerInputs(cfg, x, inp.w_r_bits, inp.bias, None),
                      flags=moe.MOE_F_FORWARD_ONLY)
    idx = to_np(layer.saved_tensor("idx"))
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert all(len(set(r)) == cfg.k for r in idx)
    assert list(idx[5]) == list(range(cfg.k))
    perm = to_np(layer.saved_tensor("perm"))
    assert np.array_equal(np.sort(perm), np.arange(cfg.T * cfg.k))
    counts = to_np(layer.saved_tensor("counts"))
    assert counts.sum() == cfg.T * cfg.k
    # every other token routes exactly as the oracle does
    L = oracle.router_logits(moe_inputs.bf16_values(x).astype(np.float64), inp.w_r)
    ok = np.isfinite(L).all(axis=1)
    assert ok.sum() == cfg.T - 2
    assert np.array_equal(idx[ok], oracle.select_topk(L[ok], cfg.k))
    assert moe.moe_device_status(layer.workspace) == moe.MOE_DEV_NONFINITE_LOGIT
    torch.cuda.synchronize()


@pytest.mark.parametrize("flags", [0, 2], ids=["direct", "ring"])
def test_forward_and_backward_do_not_block_the_host(flags):
    """moe_fwd / moe_bwd only enqueue: behind a long-running kernel on the same stream both calls
    return while the stream is still busy (no host synchronisation inside the layer), with the
    direct pull and with the ring dispatch (its rounds ordered by events between two streams)."""
    import time
    import torch
    cfg = moe_inputs.CONFIGS["tiny"].with_(backward=True)
    layer = gpu_layer(cfg, True, flags=flags)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)   # a bounded spin kernel: tens of milliseconds or more
    t0 = time.perf_counter()
    layer.forward()
    layer.backward()
    t_call = time.perf_counter() - t0
    busy = not stream.query()
    stream.synchronize()
    t_all = time.perf_counter() - t0
    log(f"host time of forward + backward calls {t_call * 1e3:.2f} ms; until the stream drained {t_all * 1e3:.1f} ms")
    assert busy, "the stream finished before the calls returned"
    assert t_call < 0.5 * t_all


def test_forward_only_matches_default_forward():
    """MOE_F_FORWARD_ONLY skips the transposed weights and changes nothing else, bit for bit."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    cfg = MID_SIG_CFG
    inp, ws, _, _, _ = oracle_layer(cfg.with_(backward=True), True)
    a = gpu_layer(cfg, False, inp=inp, ws=ws)
    b = gpu_layer(cfg, False, inp=inp, ws=ws, flags=moe.MOE_F_FORWARD_ONLY)
    assert torch.equal(a.y32, b.y32) and torch.equal(a.y, b.y)
    for name in ("hq", "hs", "g", "u", "yslot", "perm"):
        assert torch.equal(a.saved_tensor(name), b.saved_tensor(name)), name


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_unfused_forward_matches_fused_forward(cfg):
    """The unfused forward (permute, GEMM, SwiGLU pass, GEMM, unpermute, combine through HBM) is the
    in-house baseline of the fused forward: same arithmetic, so the same bits in every output and
    saved activation."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    inp = moe_inputs.layer_inputs(cfg, with_dy=False)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    fo = moe.MOE_F_FORWARD_ONLY
    a = gpu_layer(cfg, False, inp=inp, ws=ws, flags=fo)
    b = gpu_layer(cfg, False, inp=inp, ws=ws, flags=fo | moe.MOE_F_UNFUSED)
    assert torch.equal(a.y32, b.y32) and torch.equal(a.y, b.y)
    for name in ("g", "u", "hq", "hs", "yslot", "perm", "xq"):
        assert torch.equal(a.saved_tensor(name), b.saved_tensor(name)), name
    # the permuted rows are the schedule's gather of xq
    perm = b.saved_tensor("perm").long()
    R = cfg.T * cfg.k
    toks = torch.cat([perm // cfg.k, torch.arange(cfg.T, device=perm.device).repeat(cfg.n_shared)])
    assert torch.equal(b.workspace_tensor("xp"), a.saved_tensor("xq")[toks])
    assert R + cfg.n_shared * cfg.T == toks.numel()
