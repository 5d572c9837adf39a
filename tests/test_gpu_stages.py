"""Every stage of the layer on the GPU against the oracle fed the GPU's own intermediates, on the
small layers (every expert, every token): quantised weights, transposed weights W1t / W2t and the
token-axis operands bit-exact; H and [dG dU] codes bit-exact outside the float32 slack of a
rounding boundary; G, U, Y slots, y, dX slots, dx, dw, dL, dW_r, dW1, dW2 within
max |err| <= 1e-2 x RMS of the oracle tensor (stages.py states the model)."""
import pytest

from helpers import CASES, gpu_layer, log, oracle_layer  # noqa: F401
from stages import full_layer_checks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_every_stage(cfg):
    cfg = cfg.with_(backward=True)
    log(f"case {cfg.name}: inputs")
    inp, ws, _, _, _ = oracle_layer(cfg, True)
    log(f"case {cfg.name}: gpu")
    layer = gpu_layer(cfg, True, inp=inp, ws=ws)
    log(f"case {cfg.name}: stages")
    full_layer_checks(cfg, inp, ws, layer, cfg.name)


def test_every_stage_extreme_weight_blocks():
    """Weights with all-zero 32-value blocks (scale byte 0, in both the forward and the transposed
    quantisation), blocks scaled by 2^-120 (codes and scales near the bottom of their ranges) and
    by 2^20: the transposed weights stay bit-exact and every stage within its bar."""
    import numpy as np
    import moe_inputs
    cfg = moe_inputs.LayerConfig("extreme_weights", T=160, d=256, E=6, k=3, inter=256, score="softmax", seed=14,
                                 backward=True)
    inp = moe_inputs.layer_inputs(cfg, with_dy=True)
    ws = [tuple(a.copy() for a in moe_inputs.expert_weights(cfg, e)) for e in range(cfg.E)]
    ws[0][0][:32, :] = 0.0                          # gate rows 0..31 zero: zero blocks along d and along 2I
    ws[1][1][32:64, :128] = 0.0                     # W2 rows 32..63, columns 0..127: zero blocks both ways
    ws[2][0][64:96, 32:64] *= np.float32(2.0 ** -120)
    ws[3][1][:, 64:96] *= np.float32(2.0 ** -100)   # one W2 column block tiny, next to normal ones
    ws[4][0][5, :] *= np.float32(2.0 ** 20)         # one W1 row huge: its blocks dominate along 2I
    log(f"case {cfg.name}: gpu")
    layer = gpu_layer(cfg, True, inp=inp, ws=ws)
    full_layer_checks(cfg, inp, ws, layer, cfg.name)
