"""Two host threads driving the library at once.  The library's extra streams (the backward's
branch, the ring's producers and consumers) and the events that order them are kept per host
thread and device, so concurrent callers never share them.  Each thread runs forward + backward
of its own layer on its own stream, repeatedly (one with the direct pull, one through the ring);
every result is bit for bit that of the same layer run alone."""
import threading

import pytest

import moe_inputs
from helpers import MID_SIG, gpu_layer, log

pytestmark = pytest.mark.gpu

NAMES = ("y", "y32", "dx", "dx32", "dw_r", "dw1", "dw2")


def test_two_threads_on_their_own_streams():
    import torch
    import mixture_experts_layer_schedule_amd as moe
    jobs = [(moe_inputs.CONFIGS["tiny"].with_(backward=True), 0),
            (MID_SIG.with_(backward=True), moe.MOE_F_RING_DISPATCH)]
    layers = [gpu_layer(cfg, True, flags=flags) for cfg, flags in jobs]  # one step each, alone
    torch.cuda.synchronize()
    refs = [[getattr(l, n).clone() for n in NAMES] for l in layers]
    errors = []

    def work(layer):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    layer.forward(s)
                    layer.backward(s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    for l in layers:
        for n in NAMES:
            getattr(l, n).zero_()
    torch.cuda.synchronize()
    threads = [threading.Thread(target=work, args=(l,)) for l in layers]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for (cfg, _), l, ref in zip(jobs, layers, refs):
        assert moe.moe_device_status(l.workspace) == 0
        for n, r in zip(NAMES, ref):
            assert torch.equal(getattr(l, n), r), (cfg.name, n)
    log("two host threads, five steps each on their own streams: every result bit for bit")
