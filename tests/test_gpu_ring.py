"""Ring token buffers: the persistent producer/consumer gate/up kernel gives bitwise the same
results as the direct-gather kernel, at every ring capacity (down to one 256-row slot, far below
the hottest expert's load) and producer count; no token is dropped.
"""
import numpy as np
import pytest

import moe_inputs
from helpers import log, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skip(
    reason="ring dispatch disabled: the first run of its consumer on the 256-row tile core ended in a device "
           "memory fault whose cause is not identified (host emulation finds every access in bounds); "
           "the library rejects MOE_F_RING_DISPATCH until then")]

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
