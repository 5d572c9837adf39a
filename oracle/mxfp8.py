"""MXFP8 reference codec: e4m3 elements, e8m0 block scales, blocks of 32.

Test infrastructure (see the package docstring).  The pages only name the
format ("MXFP8" on a DSV3-style layer: knowledge card, section 方法/产品要点;
commentary "Cursor 开源 MoK…", section 两份成绩单).  Its arithmetic is the OCP
Microscaling v1.0 definition:

* element format e4m3 ("fn" flavour): 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits, subnormals down to 2**-9, largest finite 448, code 0x7F/0xFF
  is NaN, no infinities;
* scale format e8m0: a biased exponent byte, value 2**(byte - 127);
* a block of 32 consecutive values shares one scale
  X = 2**(floor(log2(amax)) - emax_elem) with emax_elem = 8 for e4m3;
* each element is a / X converted to e4m3 with round-to-nearest-even and
  saturation to +-448.

Readings where the format leaves a choice:
* an all-zero block takes scale byte 0 (2**-127) and zero codes;
* the exponent is clamped to the e8m0 range [-127, 127];
* the sign of a code is the sign bit of the input, so an input that rounds to
  zero keeps its sign (0x80 for negative values).

All arithmetic here is float64; inputs must already be float32 numbers (the
GPU quantises float32 values), which every caller guarantees by construction.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 value of each e4m3 code."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each value (ties to the even code); requires |v| <= 448.

    Normal range: |v| = (1 + q/8) * 2^e with e in [-6, 8], so q = rint((|v| / 2^e - 1) * 8)
    (numpy's rint rounds half to even, and the even q is the even code); q = 8 carries into the
    next binade.  Below 2^-6 the codes are the multiples q * 2^-9, q = rint(|v| * 2^9), and
    q = 8 is exactly the smallest normal (code 0x08).
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    if not np.all(mag <= E4M3_MAX):
        raise ValueError("e4m3_encode: value outside [-448, 448]")
    mant, ex = np.frexp(mag)           # mag = mant * 2^ex, 0.5 <= mant < 1 (mant = 0 for 0)
    e = ex - 1                         # mag in [2^e, 2^(e+1))
    q = np.rint((2.0 * mant - 1.0) * 8.0)
    carry = q == 8.0
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0.0, q)
    normal = ((e + 7) << 3).astype(np.int64) + q.astype(np.int64)
    sub = np.rint(mag * 2.0 ** 9).astype(np.int64)
    code = np.where(mag < 2.0 ** -6, sub, normal).astype(np.uint8)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared block exponent E_s = floor(log2 amax) - 8, clamped to [-127, 127]; -127 for amax 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)  # amax = m * 2**ex with 0.5 <= m < 1, so floor(log2 amax) = ex - 1
    es = np.clip(ex - 1 - E4M3_EMAX, -127, 127)
    return np.where(amax == 0.0, -127, es).astype(np.int64)


def _blocks(a: np.ndarray, axis: int):
    m = np.moveaxis(np.asarray(a, dtype=np.float64), axis, -1)
    n = m.shape[-1]
    if n % BLOCK:
        raise ValueError(f"quantised axis length {n} is not a multiple of {BLOCK}")
    return m, m.reshape(*m.shape[:-1], n // BLOCK, BLOCK)


def _encode_with_exponent(blocks: np.ndarray, es: np.ndarray) -> np.ndarray:
    scaled = blocks * np.exp2(-es.astype(np.float64))[..., None]
    return e4m3_encode(np.clip(scaled, -E4M3_MAX, E4M3_MAX))


def quantize(a: np.ndarray, axis: int = -1) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8-quantise ``a`` in blocks of 32 along ``axis``.

    Returns (codes uint8 with the shape of ``a``, scale bytes uint8 with the
    shape of ``a`` except ``axis`` divided by 32).
    """
    m, blocks = _blocks(a, axis)
    amax = np.max(np.abs(blocks), axis=-1)
    es = scale_exponent(amax)
    codes = _encode_with_exponent(blocks, es).reshape(m.shape)
    return np.moveaxis(codes, -1, axis), np.moveaxis((es + 127).astype(np.uint8), -1, axis)


def dequantize(q: np.ndarray, s: np.ndarray, axis: int = -1) -> np.ndarray:
    """float64 values e4m3(q) * 2**(s - 127), one scale per block of 32 along ``axis``."""
    qm = np.moveaxis(np.asarray(q, dtype=np.uint8), axis, -1)
    sm = np.moveaxis(np.asarray(s, dtype=np.uint8), axis, -1)
    n = qm.shape[-1]
    vals = e4m3_decode(qm).reshape(*qm.shape[:-1], n // BLOCK, BLOCK)
    vals = vals * np.exp2(sm.astype(np.float64) - 127.0)[..., None]
    return np.moveaxis(vals.reshape(qm.shape), -1, axis)


def requantize(q: np.ndarray, s: np.ndarray, from_axis: int, to_axis: int):
    """Dequantise along ``from_axis`` and quantise the (exact) values again along ``to_axis``."""
    return quantize(dequantize(q, s, axis=from_axis), axis=to_axis)


def quantize_range(a: np.ndarray, err: np.ndarray, axis: int = -1):
    """Admissible dequantised results when each input is only known to within ``err``.

    For every input a' with |a' - a| <= err elementwise, DQ(Q(a')) lies in the
    returned [lo, hi] (elementwise).  Used where the quantised value is computed
    from a float32 accumulation whose rounding differs between implementations:
    both sides take the rounding decision in float32, so any code inside this
    range is a correct result.  Returns (nominal DQ(Q(a)), lo, hi).
    """
    m, blocks = _blocks(a, axis)
    e = np.broadcast_to(np.asarray(err, dtype=np.float64), np.shape(a))
    em = np.moveaxis(e, axis, -1).reshape(blocks.shape)
    mag = np.abs(blocks)
    amax_lo = np.max(np.maximum(mag - em, 0.0), axis=-1)
    amax_hi = np.max(mag + em, axis=-1)
    es_nom = scale_exponent(np.max(mag, axis=-1))
    es_lo = scale_exponent(amax_lo)
    es_hi = scale_exponent(amax_hi)
    nominal = e4m3_decode(_encode_with_exponent(blocks, es_nom)) * np.exp2(es_nom)[..., None]
    lo = nominal.copy()
    hi = nominal.copy()
    span = int(np.max(es_hi - es_lo)) if es_hi.size else 0
    for step in range(span + 1):
        es = np.minimum(es_lo + step, es_hi)
        f = np.exp2(es.astype(np.float64))[..., None]
        lo = np.minimum(lo, e4m3_decode(_encode_with_exponent(blocks - em, es)) * f)
        hi = np.maximum(hi, e4m3_decode(_encode_with_exponent(blocks + em, es)) * f)

    def back(v):
        return np.moveaxis(v.reshape(m.shape), -1, axis)

    return back(nominal), back(lo), back(hi)
