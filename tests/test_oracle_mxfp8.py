"""Pins of the oracle's MXFP8 codec against things other than itself.

* hand values worked from the OCP MX v1.0 definition (tests/golden/mxfp8_hand_values.txt);
* torch's float8_e4m3fn codec (a library routine) for every code and for random inputs;
* closed forms: powers of two, round trips of on-grid values, the half-ulp bound.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_hand_values.txt")


def _num(tok: str) -> float:
    if "*2^" in tok:
        a, b = tok.split("*2^")
        return float(a) * 2.0 ** int(b)
    return float(np.float32(float(tok)))


def _golden_cases():
    cases = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        amax, value, scale, code, dq = line.split()
        cases.append((_num(amax), _num(value), int(scale, 16), int(code, 16), _num(dq)))
    return cases


@pytest.mark.parametrize("amax,value,scale,code,dq", _golden_cases())
def test_hand_values(amax, value, scale, code, dq):
    block = np.zeros(32)
    block[0] = amax
    block[1] = value
    q, s = oracle.quantize(block[None, :], axis=1)
    assert s.shape == (1, 1)
    assert int(s[0, 0]) == scale
    assert int(q[0, 1]) == code
    back = oracle.dequantize(q, s, axis=1)
    assert back[0, 1] == dq


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_matches_torch_float8_rne():
    rng = np.random.default_rng(7)
    # values spread over the whole e4m3 range, plus exact midpoints and grid points
    mags = np.exp2(rng.uniform(-12, math.log2(448.0), size=200_000))
    grid = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    v = np.concatenate([mags, grid, mids, -mags[:1000], -mids, [0.0, -0.0]]).astype(np.float32)
    ours = oracle.e4m3_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0]))


@pytest.mark.parametrize("p", [-126, -20, -8, -1, 0, 1, 5, 8, 100, 127])
def test_scale_exponent_powers_of_two(p):
    for m in (1.0, 1.5, 1.999):
        amax = m * 2.0 ** p
        assert int(oracle.scale_exponent(np.array(amax))) == max(-127, min(127, p - 8))
    assert int(oracle.scale_exponent(np.array(0.0))) == -127


def test_scale_puts_block_max_in_top_binade():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))).astype(np.float32)
    q, s = oracle.quantize(a.astype(np.float64), axis=1)
    blocks = np.abs(a.astype(np.float64)).reshape(64, 8, 32)
    amax = blocks.max(axis=2)
    scaled = amax / np.exp2(s.astype(np.float64) - 127)
    assert np.all((scaled >= 256) & (scaled < 512))


def test_round_trip_on_grid_is_exact():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(16, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x42  # no NaN codes
    # force every block's max magnitude into the top binade so re-quantising keeps the scale
    codes[:, ::32] = 0x7E
    scales = rng.integers(100, 140, size=(16, 4)).astype(np.uint8)
    vals = oracle.dequantize(codes, scales, axis=1)
    q2, s2 = oracle.quantize(vals, axis=1)
    assert np.array_equal(s2, scales)
    assert np.array_equal(oracle.dequantize(q2, s2, axis=1), vals)


def test_half_ulp_error_bound():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((32, 512)).astype(np.float32).astype(np.float64)
    q, s = oracle.quantize(a, axis=1)
    back = oracle.dequantize(q, s, axis=1)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    scaled = np.abs(a) / scale
    # ulp of e4m3 at each scaled magnitude (subnormal spacing below 2^-6)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(scaled, 2.0 ** -9))), -6) - 3) * scale
    sat = scaled > 448
    assert np.all(np.abs(back - a)[~sat] <= ulp[~sat] / 2)
    assert np.all(np.abs(back[sat]) == 448 * scale[sat])


def test_quantize_along_axis0_is_transpose_of_axis1():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((64, 96)).astype(np.float32).astype(np.float64)
    q0, s0 = oracle.quantize(a, axis=0)
    q1, s1 = oracle.quantize(a.T, axis=1)
    assert np.array_equal(q0, q1.T) and np.array_equal(s0, s1.T)
    assert s0.shape == (2, 96)


def test_quantize_range_contains_perturbed_results():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((8, 256)).astype(np.float32).astype(np.float64)
    err = np.abs(a) * 1e-3 + 1e-6
    nom, lo, hi = oracle.quantize_range(a, err, axis=1)
    q, s = oracle.quantize(a, axis=1)
    assert np.array_equal(nom, oracle.dequantize(q, s, axis=1))
    assert np.all(lo <= nom) and np.all(nom <= hi)
    for _ in range(20):
        ap = a + err * rng.uniform(-1, 1, size=a.shape)
        ap = ap.astype(np.float32).astype(np.float64)
        ap = np.clip(ap, a - err, a + err)
        qp, sp = oracle.quantize(ap, axis=1)
        dp = oracle.dequantize(qp, sp, axis=1)
        assert np.all(dp >= lo) and np.all(dp <= hi)
    # no uncertainty: the range collapses to the nominal result
    nom0, lo0, hi0 = oracle.quantize_range(a, 0.0, axis=1)
    assert np.array_equal(lo0, nom0) and np.array_equal(hi0, nom0)


def test_requantize_other_axis():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    q, s = oracle.quantize(a, axis=1)
    q2, s2 = oracle.requantize(q, s, from_axis=1, to_axis=0)
    exact = oracle.dequantize(q, s, axis=1)
    q3, s3 = oracle.quantize(exact, axis=0)
    assert np.array_equal(q2, q3) and np.array_equal(s2, s3)
    assert mxfp8.BLOCK == 32


def test_quantize_range_is_attained():
    """Tightness of the admissible range: with a few uncertain values in a block, every bound
    quantize_range reports is the result of some perturbation within the error (brute force over
    the 3^m corner perturbations), and every corner result lies inside the bounds."""
    import itertools
    rng = np.random.default_rng(11)
    for trial in range(40):
        a = (rng.standard_normal(32) * 2.0 ** rng.integers(-3, 4)).astype(np.float32).astype(np.float64)
        unc = rng.choice(32, size=3, replace=False)
        if trial % 2:
            unc[0] = int(np.argmax(np.abs(a)))       # the block maximum itself uncertain
        err = np.zeros(32)
        err[unc] = np.abs(a[unc]) * 2.0 ** -rng.integers(3, 7, size=3)
        nom, lo, hi = oracle.quantize_range(a[None], err[None], axis=1)
        results = []
        for signs in itertools.product((-1.0, 0.0, 1.0), repeat=3):
            b = a.copy()
            b[unc] += np.array(signs) * err[unc]
            q, s = oracle.quantize(b[None], axis=1)
            results.append(oracle.dequantize(q, s, axis=1)[0])
        results = np.array(results)
        assert np.all(results >= lo[0]) and np.all(results <= hi[0])
        # attained: for the uncertain values and every value whose bound moved
        moved = np.where((lo[0] != nom[0]) | (hi[0] != nom[0]))[0]
        for i in set(moved.tolist()) | set(unc.tolist()):
            assert results[:, i].min() == lo[0, i] and results[:, i].max() == hi[0, i], (trial, i)
