"""Every stage of the layer on the GPU against the oracle fed the GPU's own intermediates, on the
small layers (every expert, every token): quantised weights, transposed weights W1t / W2t and the
token-axis operands bit-exact; H and [dG dU] codes bit-exact outside the float32 slack of a
rounding boundary; G, U, Y slots, y, dX slots, dx, dw, dL, dW_r, dW1, dW2 within
max |err| <= 1e-2 x RMS of the oracle tensor (stages.py states the model)."""
import pytest

from helpers import CASES, gpu_layer, log, oracle_layer
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
