"""MXFP8 kernels against the oracle, bit for bit."""
import numpy as np
import pytest

import moe_inputs
import oracle
from helpers import log

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _quant_gpu(a: np.ndarray, is_f32: bool):
    torch = _torch()
    import mixture_experts_layer_schedule_amd as moe

    rows, cols = a.shape
    if is_f32:
        src = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    else:
        src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(src, 1 if is_f32 else 0, rows, cols, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def test_quant_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = moe_inputs.bf16_values(bits)
    keep = np.isfinite(vals)
    bits = bits[keep]
    bits = bits[: bits.size // 32 * 32]
    rng = np.random.default_rng(0)
    for trial in range(3):  # three block arrangements of the same patterns
        b = bits if trial == 0 else rng.permutation(bits)
        a = b.reshape(-1, 32)
        log(f"quant bf16 patterns: trial {trial}, {a.shape}")
        q, s = _quant_gpu(a, is_f32=False)
        rq, rs = oracle.quantize(moe_inputs.bf16_values(a).astype(np.float64), axis=1)
        assert np.array_equal(s, rs)
        assert np.array_equal(q, rq)


def test_quant_bf16_activations_and_f32_weights():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((257, 512)) * np.exp2(rng.integers(-40, 40, size=(257, 1)))).astype(np.float32)
    xb = moe_inputs.bf16_bits(x)
    q, s = _quant_gpu(xb, is_f32=False)
    rq, rs = oracle.quantize(moe_inputs.bf16_values(xb).astype(np.float64), axis=1)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)
    w = (rng.standard_normal((384, 1024)) / 32.0).astype(np.float32)
    w[3, :64] = 0.0  # all-zero blocks
    w[5, 32:64] = -0.0
    q, s = _quant_gpu(w, is_f32=True)
    rq, rs = oracle.quantize(w.astype(np.float64), axis=1)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


@pytest.mark.parametrize("batch,rows,cols", [(3, 192, 128), (2, 256, 384)])
def test_requant_transpose(batch, rows, cols):
    """Both tilings: 64 x 64 (shapes that are not multiples of 128) and 128 x 128."""
    torch = _torch()
    import mixture_experts_layer_schedule_amd as moe

    rng = np.random.default_rng(2)
    w = (rng.standard_normal((batch, rows, cols)) * np.exp2(rng.integers(-8, 8, size=(batch, rows, 1)))).astype(
        np.float32)
    w[0, :32, :32] = 0.0                      # an all-zero block (scale byte 0) on both sides
    w[-1, 32:64, :] *= np.float32(2.0 ** -120)  # tiny values: scale bytes near the bottom of the range
    rq, rs = oracle.quantize(w.astype(np.float64), axis=2)
    q = torch.from_numpy(rq).cuda()
    s = torch.from_numpy(rs).cuda()
    qt = torch.empty((batch, cols, rows), dtype=torch.uint8, device="cuda")
    st = torch.empty((batch, cols, rows // 32), dtype=torch.uint8, device="cuda")
    moe.moe_requant_transpose(q, s, batch, rows, cols, qt, st)
    torch.cuda.synchronize()
    eq, es = oracle.requantize(rq, rs, from_axis=2, to_axis=1)  # [batch, rows, cols] blocks along rows
    assert np.array_equal(qt.cpu().numpy(), eq.transpose(0, 2, 1))
    assert np.array_equal(st.cpu().numpy(), es.transpose(0, 2, 1))
