"""The layer on the GPU against the oracle on the same seeded inputs.

Bit-exact: top-k selection, schedule (counts, offsets, permutation, inverse), quantised x.
Within tolerance (max |err| <= 1e-2 x RMS of the oracle tensor, on the float32 copies):
y, dx, dW_router, dW1, dW2; the bf16 outputs equal the float32 copies rounded to nearest even.
Bitwise identical across runs.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
from helpers import gpu_layer, log, oracle_layer, rel_err, rms, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2

MID = moe_inputs.LayerConfig("mid", T=512, d=512, E=16, k=4, inter=256, score="softmax", seed=7)
MID_SIG = moe_inputs.LayerConfig("mid_sig_shared", T=384, d=256, E=24, k=6, inter=384, score="sigmoid", seed=8,
                                 n_shared=1, zipf_s=1.1, zipf_lam=0.5)
CASES = [moe_inputs.CONFIGS["tiny"], MID, MID_SIG]


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


def test_gate_up_and_h(pair):
    cfg, inp, fw, bw, layer = pair
    G = to_np(layer.saved_tensor("g")).astype(np.float64)
    U = to_np(layer.saved_tensor("u")).astype(np.float64)
    Gr, Ur = _expert_rows(fw, "G"), _expert_rows(fw, "U")
    eg, eu = rel_err(G, Gr), rel_err(U, Ur)
    log(f"{cfg.name}: G err/rms {eg:.2e}  U err/rms {eu:.2e}")
    assert eg < 1e-4 and eu < 1e-4
    hq = to_np(layer.saved_tensor("hq"))
    hs = to_np(layer.saved_tensor("hs"))
    Hr = _expert_rows(fw, "Hq")
    frac = np.mean(hq != Hr)
    log(f"{cfg.name}: H codes differing from the oracle: {frac:.2e}, scales: {np.mean(hs != _expert_rows(fw, 'Hs')):.2e}")
    assert frac < 1e-3


def test_forward_output(pair):
    cfg, inp, fw, bw, layer = pair
    y32 = to_np(layer.y32).astype(np.float64)
    e = rel_err(y32, fw.y)
    log(f"{cfg.name}: y max|err|/rms = {e:.3e}")
    assert e <= TOL
    assert np.array_equal(to_np(layer.y.view(__import__('torch').int16)), _bf16_rne(to_np(layer.y32)))
    ys = to_np(layer.saved_tensor("yslot"))
    assert rel_err(ys[:, : cfg.k].reshape(-1, cfg.d), fw.Yrows[fw.sched.pos.reshape(-1)]) <= TOL


def test_backward_outputs(pair):
    cfg, inp, fw, bw, layer = pair
    import torch
    res = {}
    res["dx"] = rel_err(to_np(layer.dx32), bw.dx)
    res["dw_router"] = rel_err(to_np(layer.dw_r), bw.dw_r)
    dw1 = to_np(layer.dw1)
    dw2 = to_np(layer.dw2)
    NX = cfg.E + cfg.n_shared
    ref1 = np.stack([bw.dW1[e] for e in range(NX)])
    ref2 = np.stack([bw.dW2[e] for e in range(NX)])
    res["dW1"] = rel_err(dw1, ref1)
    res["dW2"] = rel_err(dw2, ref2)
    log(f"{cfg.name}: backward max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in res.items()))
    assert np.array_equal(to_np(layer.dx.view(torch.int16)), _bf16_rne(to_np(layer.dx32)))
    for k, v in res.items():
        assert v <= TOL, k


def test_bitwise_reproducible(pair):
    cfg, inp, fw, bw, layer = pair
    import torch
    y0 = layer.y32.clone()
    dx0 = layer.dx32.clone()
    dw10 = layer.dw1.clone()
    for _ in range(3):
        layer.forward()
        layer.backward()
    torch.cuda.synchronize()
    assert torch.equal(y0, layer.y32)
    assert torch.equal(dx0, layer.dx32)
    assert torch.equal(dw10, layer.dw1)
