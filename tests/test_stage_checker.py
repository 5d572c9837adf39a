"""The stage checker (tests/stages.py) accepts a layer built from the oracle's own intermediates and
rejects planted mistakes, all on the CPU (the GPU tests rely on it)."""
import numpy as np
import pytest

import moe_inputs
from fake_layer import FakeLayer
from stages import full_layer_checks

CASES = [
    moe_inputs.LayerConfig("small", T=40, d=128, E=4, k=2, inter=128, score="softmax", seed=21, backward=True),
    moe_inputs.LayerConfig("small_shared", T=33, d=256, E=6, k=2, inter=128, score="sigmoid", seed=22,
                           n_shared=1, zipf_s=1.1, zipf_lam=1.0, backward=True),
    moe_inputs.LayerConfig("one_token", T=1, d=256, E=8, k=2, inter=128, score="sigmoid", seed=23, n_shared=1,
                           backward=True),
]


def _fake(cfg):
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    ws = [moe_inputs.expert_weights(cfg, e) for e in range(cfg.E + cfg.n_shared)]
    return inp, ws, FakeLayer(cfg, inp, ws)


@pytest.fixture(scope="module", params=CASES, ids=lambda c: c.name)
def fake(request):
    cfg = request.param
    return (cfg,) + _fake(cfg)


def test_checker_accepts_the_oracle(fake):
    cfg, inp, ws, layer = fake
    full_layer_checks(cfg, inp, ws, layer, cfg.name)


def _expect_failure(cfg, inp, ws, layer, plant):
    undo = plant(layer)
    try:
        with pytest.raises(AssertionError):
            full_layer_checks(cfg, inp, ws, layer, cfg.name)
    finally:
        undo()


def _swap(t, new):
    old = t.clone()
    t.copy_(new)
    return lambda: t.copy_(old)


def test_checker_rejects_planted_mistakes(fake):
    cfg, inp, ws, layer = fake
    e = int(np.argmax(layer.saved_tensor("counts").numpy()[:cfg.E]))
    lo = int(layer.saved_tensor("offsets")[e])
    t1, t2 = min(1, cfg.T - 1), min(2, cfg.T - 1)
    plants = {
        # W1t requantised along the wrong axis (blocks along d instead of 2I): codes differ
        "w1t axis": lambda L: _swap(L.saved_tensor("w1t")[e], L.w1q[e].T.contiguous()),
        # one H code moved to its neighbour where the code is unique
        "h code": lambda L: _swap(L.saved_tensor("hq")[lo, :1], (L.saved_tensor("hq")[lo, :1] ^ 2)),
        # a Y slot row scaled by 2 %
        "y slot": lambda L: _swap(L.saved_tensor("yslot")[0, 0], L.saved_tensor("yslot")[0, 0] * 1.02),
        # [dG dU] scale byte of one block off by one
        "dgu scale": lambda L: _swap(L.workspace_tensor("dgus")[lo, :1], L.workspace_tensor("dgus")[lo, :1] + 1),
        # token-axis X operand of the expert quantised with one scale byte too large
        "xt scale": lambda L: _swap(L.workspace_tensor("xts")[:1, :1], L.workspace_tensor("xts")[:1, :1] + 1),
        # dW1 of the expert transposed wrong: gate and up halves swapped
        "dw1 halves": lambda L: _swap(L.dw1[e], L.dw1[e].roll(cfg.inter, dims=0)),
        # dx missing the router term of one token
        "dx": lambda L: _swap(L.dx32[t1], L.dx32[t1] * 0.9),
        # the combine weights of one token swapped
        "w": lambda L: _swap(L.saved_tensor("w")[t2], L.saved_tensor("w")[t2].flip(0)),
    }
    for name, plant in plants.items():
        _expect_failure(cfg, inp, ws, layer, plant)
