"""Graph capture of a whole layer step.  moe_fwd and moe_bwd only enqueue kernels, plus event
record / wait pairs between the caller's stream and the library's own streams (the backward's
second-stream branch, the ring's producers).  There is no memset, no allocation and no host
synchronisation, so a caller can capture forward + backward into a HIP graph and replay it.
Every replay, with eager work and synchronisations between replays, reproduces the eager step
bit for bit."""
import pytest

import moe_inputs
from helpers import gpu_layer, log

pytestmark = pytest.mark.gpu

NAMES = ("y", "y32", "dx", "dx32", "dw_r", "dw1", "dw2")


@pytest.mark.parametrize("flags", [0, 2, 4], ids=["two-stream", "ring", "launch-order"])
def test_captured_step_replays_bitwise(flags):
    import torch
    cfg = moe_inputs.CONFIGS["tiny"].with_(backward=True)
    layer = gpu_layer(cfg, True, flags=flags)  # one eager step: streams and events exist now
    outs = lambda: [getattr(layer, n) for n in NAMES]  # noqa: E731
    ref = [t.clone() for t in outs()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # a warm-up step on a side stream, as graph capture expects
        layer.forward()
        layer.backward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward()
        layer.backward()
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs():
            t.zero_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, r, t in zip(NAMES, ref, outs()):
            assert torch.equal(r, t), f"replay {i}: {name}"
    log(f"graph of one forward + backward step replayed 3 times bit for bit (flags {flags})")
    del g
