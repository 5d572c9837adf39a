"""Ring token buffers (MOE_F_RING_DISPATCH): producer workgroups on a second stream gather each
round of chunks (GEMM row tiles) into the fixed-capacity ring while the gate/up GEMM (forward)
or the dgrad-down GEMM (backward, dY rows) runs the previous round from it, ordered by events.  The results are bitwise those of direct gather at
every ring capacity (down to one slot, far below the hottest expert's load, so the ring wraps
many times) and producer count; no row is dropped.
"""
import numpy as np
import pytest

import moe_inputs
from helpers import EMPTY, K1_SHARED, MAX_ROUTE, ONE_TOKEN, RAGGED, log, to_np

EDGE = {c.name: c for c in (ONE_TOKEN, EMPTY, MAX_ROUTE, K1_SHARED, RAGGED)}

pytestmark = pytest.mark.gpu

SKEW = moe_inputs.LayerConfig("skew", T=1024, d=256, E=32, k=4, inter=256, score="sigmoid", seed=9,
                              n_shared=1, zipf_s=1.1, zipf_lam=1.5)


def _run(cfg, inp, ws, **kw):
    import torch
    from mixture_experts_layer_schedule_amd import MoeLayer
    import mixture_experts_layer_schedule_amd as moe

    layer = MoeLayer.from_config(cfg, with_backward=False, **kw)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias)
    layer.load_experts((e, w1, w2) for e, (w1, w2) in enumerate(ws))
    layer.forward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(layer.workspace) == 0
    return layer


RING = 2  # MOE_F_RING_DISPATCH
WIDE = moe_inputs.LayerConfig("wide", T=512, d=384, E=12, k=3, inter=640, score="softmax", seed=10)


@pytest.fixture(scope="module", params=[SKEW, WIDE], ids=lambda c: c.name)
def skew(request):
    cfg = request.param
    inp = moe_inputs.layer_inputs(cfg)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    import mixture_experts_layer_schedule_amd as moe
    ref = _run(cfg, inp, ws, flags=moe.MOE_F_DIRECT_GATHER)
    counts = to_np(ref.saved_tensor("counts"))
    log(f"skewed loads: max {counts[:cfg.E].max()} rows, mean {counts[:cfg.E].mean():.0f}")
    return cfg, inp, ws, ref


@pytest.mark.parametrize("ring_rows,producers", [(256, 1), (512, 3), (768, 16), (1024, 8), (8192, 32)])
def test_ring_matches_direct_gather(skew, ring_rows, producers):
    cfg, inp, ws, ref = skew
    counts = to_np(ref.saved_tensor("counts"))
    layer = _run(cfg, inp, ws, ring_rows=ring_rows, producer_wgs=producers, flags=RING)
    if ring_rows < counts.max():
        log(f"ring {ring_rows} rows < peak load {counts.max()}: wraps")
    for name in ("g", "u", "hq", "hs", "yslot"):
        assert np.array_equal(to_np(layer.saved_tensor(name)), to_np(ref.saved_tensor(name))), name
    assert np.array_equal(to_np(layer.y32), to_np(ref.y32))


def test_every_row_processed(skew):
    """Each permuted row got a gate/up result (no row dropped): G rows are all written."""
    cfg, inp, ws, ref = skew
    layer = _run(cfg, inp, ws, ring_rows=256, producer_wgs=2, flags=RING)
    g = layer.saved_tensor("g")
    g.zero_()
    layer.forward()
    import torch
    torch.cuda.synchronize()
    rows = to_np(g)
    assert np.all(np.any(rows != 0, axis=1)), "a routed row was not processed"
    assert rows.shape[0] == cfg.rows


@pytest.mark.parametrize("chunk_rows,ring_rows", [(128, 128), (96, 480), (64, 4096)])
def test_ring_with_shorter_chunks(skew, chunk_rows, ring_rows):
    """Slots of chunk_rows rows (the row-tile height): still the direct-gather bits."""
    cfg, inp, ws, ref = skew
    layer = _run(cfg, inp, ws, ring_rows=ring_rows, chunk_rows=chunk_rows, producer_wgs=4, flags=RING)
    for name in ("g", "u", "hq", "hs", "yslot"):
        assert np.array_equal(to_np(layer.saved_tensor(name)), to_np(ref.saved_tensor(name))), name


def _run_bwd(cfg, inp, ws, **kw):
    import torch
    from mixture_experts_layer_schedule_amd import MoeLayer
    import mixture_experts_layer_schedule_amd as moe

    layer = MoeLayer.from_config(cfg, with_backward=True, **kw)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits)
    layer.load_experts((e, w1, w2) for e, (w1, w2) in enumerate(ws))
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(layer.workspace) == 0
    return layer


def _bwd_results(layer):
    import torch
    out = {"dx": layer.dx.view(torch.int16), "dx32": layer.dx32, "dw_r": layer.dw_r, "dw1": layer.dw1, "dw2": layer.dw2}
    for n in ("dguq", "dgus"):
        out[n] = layer.workspace_tensor(n)
    return {n: to_np(t) for n, t in out.items()}


@pytest.fixture(scope="module", params=[SKEW, WIDE], ids=lambda c: c.name)
def bwd_ref(request):
    import mixture_experts_layer_schedule_amd as moe
    cfg = request.param.with_(backward=True)
    inp = moe_inputs.layer_inputs(cfg)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    return cfg, inp, ws, _bwd_results(_run_bwd(cfg, inp, ws, flags=moe.MOE_F_DIRECT_GATHER))


@pytest.mark.parametrize("ring_rows,producers,serial", [(256, 1, False), (512, 3, True), (768, 16, False),
                                                        (8192, 32, True)])
def test_backward_ring_matches_direct_pull(bwd_ref, ring_rows, producers, serial):
    """The backward's pull reverse-combine through the ring (dY rows staged in the slots for the
    dgrad-down GEMM), with the producers on their own stream beside the backward's second-stream
    branch or everything in launch order: [dG dU] codes and scales and every gradient bitwise
    those of the direct pull."""
    import mixture_experts_layer_schedule_amd as moe
    cfg, inp, ws, ref = bwd_ref
    flags = RING | (moe.MOE_F_SERIAL_BWD if serial else 0)
    got = _bwd_results(_run_bwd(cfg, inp, ws, ring_rows=ring_rows, producer_wgs=producers, flags=flags))
    for n, v in ref.items():
        assert np.array_equal(got[n], v), n


@pytest.mark.parametrize("cfg", [EDGE[n] for n in ("one_token", "empty_experts", "max_route", "k1_shared", "ragged")],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("ring_rows", [256, 512])
def test_ring_on_edge_layers(cfg, ring_rows):
    """The edge layers (one token, experts with no rows, E = 512 with k = 16, k = 1 plus a shared
    expert, ragged tails) through a one-slot and a two-slot ring, forward and backward: every
    output, gradient and [dG dU] bit for bit those of the direct pull."""
    import mixture_experts_layer_schedule_amd as moe
    cfg = cfg.with_(backward=True)
    inp = moe_inputs.layer_inputs(cfg)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    ref = _bwd_results(_run_bwd(cfg, inp, ws, flags=moe.MOE_F_DIRECT_GATHER))
    got = _bwd_results(_run_bwd(cfg, inp, ws, ring_rows=ring_rows, flags=RING))
    for n, v in ref.items():
        assert np.array_equal(got[n], v), n


def test_ring_tuner_keeps_the_bits(bwd_ref):
    """The tuner over the ring's knobs (row-tile height, producer workgroups, capacities up to the
    configured one) runs every candidate in the layer's one workspace and leaves the fastest in
    its configuration; the tuned layer still computes the direct pull's bits."""
    import torch
    from mixture_experts_layer_schedule_amd import tune
    cfg, inp, ws, ref = bwd_ref
    layer = _run_bwd(cfg, inp, ws, ring_rows=1024, flags=RING)
    res = tune.tune(layer, backward=True, steps=1, warmup=1)
    cands = tune.candidates(layer.T, layer.E, layer.k, layer.S, True, 1024)
    assert res.best in cands and set(res.ms) == set(cands)
    assert {kn.ring_rows for kn in cands} == {1024, 512, 256}
    log("ring tuner: " + ", ".join(f"{k} {v:.3f}" for k, v in list(res.table().items())[:6]))
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    got = _bwd_results(layer)
    for n, v in ref.items():
        assert np.array_equal(got[n], v), n


def test_kimi_shape_ring_below_peak_load():
    """The Kimi-K2-shaped skewed workload (16,384 tokens, 384 + 1 experts, the hottest expert far
    above the mean) at its own ring capacity of 2,048 rows, below the hottest expert's load:
    every output and saved activation bitwise equal to direct gather."""
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import MoeLayer
    cfg = moe_inputs.CONFIGS["kimi_k2_skew"]
    inp = moe_inputs.layer_inputs(cfg)
    layer = MoeLayer.from_config(cfg, with_backward=False, ring_rows=cfg.ring_rows, producer_wgs=32, flags=RING)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias)
    log("kimi: drawing and quantising the experts")
    layer.load_experts(moe_inputs.iter_expert_weights(cfg, threads=16))
    layer.forward()
    torch.cuda.synchronize()
    assert moe.moe_device_status(layer.workspace) == 0
    counts = to_np(layer.saved_tensor("counts"))
    log(f"kimi: hottest expert {counts.max()} rows, ring {cfg.ring_rows} rows")
    assert counts.max() > cfg.ring_rows
    names = ("g", "u", "hq", "hs", "yslot")
    ring = {n: layer.saved_tensor(n).clone() for n in names}
    ring["y"] = layer.y32.clone()
    layer.cfg.flags, layer.cfg.ring_rows, layer.cfg.producer_wgs = moe.MOE_F_DIRECT_GATHER, 0, 0
    layer.forward()
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(ring[n], layer.saved_tensor(n)), n
    assert torch.equal(ring["y"], layer.y32)


@pytest.mark.skip(reason="the persistent producer/consumer kernel (csrc/ring.hip) is not launched: its first run "
                         "on the 256-row tile core ended in a device memory fault whose cause is not identified; "
                         "MOE_F_RING_DISPATCH runs the stream-ordered ring instead")
def test_persistent_ring_kernel():
    pass
