"""Shared pieces of the GPU tests: run the library and the oracle on the same seeded inputs."""
from __future__ import annotations

import functools
import sys

import numpy as np

import moe_inputs
import oracle


# Small layers checked whole: the tiny workload, two mid-size layers (one with a shared expert and
# a Zipf router bias) and edge cases:
MID = moe_inputs.LayerConfig("mid", T=512, d=512, E=16, k=4, inter=256, score="softmax", seed=7)
MID_SIG = moe_inputs.LayerConfig("mid_sig_shared", T=384, d=256, E=24, k=6, inter=384, score="sigmoid", seed=8,
                                 n_shared=1, zipf_s=1.1, zipf_lam=0.5)
# a ragged token count (not a multiple of any tile or block) with 12 experts; a
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
# one token (two routed rows and a shared row; every other expert empty)
ONE_TOKEN = moe_inputs.LayerConfig("one_token", T=1, d=256, E=8, k=2, inter=128, score="sigmoid", seed=14,
                                   n_shared=1)
CASES = [moe_inputs.CONFIGS["tiny"], MID, MID_SIG, RAGGED, EMPTY, K_EQ_E, K1_SHARED, MAX_ROUTE, ONE_TOKEN]


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
