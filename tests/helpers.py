"""Shared pieces of the GPU tests: run the library and the oracle on the same seeded inputs."""
from __future__ import annotations

import functools
import sys

import numpy as np

import moe_inputs
import oracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def oracle_layer(cfg: moe_inputs.LayerConfig, backward: bool):
    inp = moe_inputs.layer_inputs(cfg, with_dy=backward)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    ex = oracle.oracle_experts([w[0] for w in ws], [w[1] for w in ws])
    fw = oracle.layer_forward(inp.x, inp.w_r, ex, cfg.k, cfg.score, inp.bias, cfg.n_shared)
    bw = oracle.layer_backward(fw, inp.dy, inp.x, inp.w_r, ex, cfg.score) if backward else None
    return inp, ws, ex, fw, bw


def gpu_layer(cfg: moe_inputs.LayerConfig, backward: bool, inp=None, ws=None, **kw):
    import torch
    from mixture_experts_layer_schedule_amd import MoeLayer

    if inp is None:
        inp = moe_inputs.layer_inputs(cfg, with_dy=backward)
    layer = MoeLayer.from_config(cfg, with_backward=backward, **kw)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, inp.dy_bits if backward else None)
    if ws is None:
        layer.load_experts(moe_inputs.iter_expert_weights(cfg))
    else:
        layer.load_experts((e, w1, w2) for e, (w1, w2) in enumerate(ws))
    log(f"  {cfg.name}: forward")
    layer.forward()
    torch.cuda.synchronize()
    if backward:
        log(f"  {cfg.name}: backward")
        layer.backward()
        torch.cuda.synchronize()
    return layer


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def rel_err(got, ref) -> float:
    """max |got - ref| / rms(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    r = rms(ref)
    return float(np.max(np.abs(got - ref))) / r if r > 0 else float(np.max(np.abs(got - ref)))


def to_np(t):
    return t.detach().cpu().numpy()
