"""MXFP8 quantiser of the oracle: E4M3 elements with one E8M0 scale per 32.

Test infrastructure only: nothing in the GPU library imports this module.

The pages say only that MXFP8 activation quantisation is fused into the
dispatch, grouped-GEMM and SwiGLU data paths (kucoin.com news flash "O MoK do
Cursor alcança aumento de desempenho de 2,37x no NVIDIA GB300 NVL72",
section 02; deepdigest.ru article on MoK).  The format itself is the OCP
Microscaling one: a block of 32 values shares a power-of-two scale stored as
an 8-bit biased exponent (E8M0, bias 127), and each value is an FP8 E4M3
number (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
max normal 448, S.1111.111 is NaN).

Conversion of one block v[0..31] (the reading used throughout):
  amax = max |v_i|
  amax == 0  ->  scale code 0, every element code 0
  otherwise  s = clamp(floor(log2 amax) - 8, -127, 127)   (8 = E4M3's emax)
             scale code = s + 127
             q_i = E4M3(clamp(v_i * 2^-s, -448, 448)), nearest, ties to even,
                   gradual underflow into the subnormals (quantum 2^-9)
  dequantised value = E4M3value(q_i) * 2^s (exact in fp32 and bf16)
The sign bit of a code is set exactly when the value is < 0, so a negative
value that rounds to zero keeps a sign (0x80) and +0/-0 inputs give 0x00.

Lower-precision element formats of the same specification (the pages mention
4-bit expert kernels, noticiai.com.br "Cursor abre código do
Mixture-of-Kittens", section "Por que a camada MoE virou o gargalo"; the MX
family is their counterpart here): FP6 E2M3 (bias 1, max 7.5), FP6 E3M2
(bias 3, max 28) and FP4 E2M1 (bias 1, max 6).  None has infinities or NaNs;
the conversion is the same with the format's own emax (2, 4 and 2):
s = clamp(floor(log2 amax) - emax, -127, 127), elements clamped to the
format's maximum and rounded to nearest, ties to even, with gradual
underflow.  A code is sign | exponent field | mantissa, one code per byte.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_encode(v) -> np.ndarray:
    """Encode values with |v| <= 448 to E4M3 codes (uint8), nearest-even.

    A value in the binade [2^e, 2^(e+1)) (e >= -6) is a multiple of the
    quantum 2^(e-3); below the smallest normal 2^-6 the quantum stays the
    subnormal one, 2^-9, so the binade exponent is floored at -6.  With
    q = |v| / 2^(e-3) rounded to the nearest integer (ties to even), q lies
    in [8, 16] for a normal and in [0, 8] below the normals, and the code's
    low seven bits are 8 (e + 6) + q: exponent field e + 7 with mantissa
    q - 8 for a normal, the subnormal mantissa q itself when e = -6, and a
    q of 16 (or of 8 from below the normals) is the next binade's
    mantissa 0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode: value outside [-448, 448]")
    _, ex = np.frexp(np.maximum(a, 2.0 ** -7))   # a = m 2^ex with m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    q = np.rint(np.ldexp(a, 3 - e)).astype(np.int64)
    code = 8 * (e + 6) + q
    code |= (v < 0).astype(np.int64) << 7
    return code.astype(np.uint8)


def _e4m3_value(code) -> np.ndarray:
    """Value of E4M3 codes from their bit fields (fp64); NaN codes give NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(ex == 0, np.ldexp(man.astype(np.float64), -9),
                   np.ldexp((8 + man).astype(np.float64), ex - 10))
    mag = np.where((ex == 15) & (man == 7), np.nan, mag)
    return sign * mag


_E4M3_VALUES = _e4m3_value(np.arange(256))


def e4m3_decode(code) -> np.ndarray:
    """Value of E4M3 codes (fp64): a lookup in the table of all 256 codes
    built from the bit fields; the NaN codes decode to NaN."""
    return _E4M3_VALUES[np.asarray(code, dtype=np.uint8)]


class ElementFormat:
    """An MX element format: sign, `ebits` exponent bits with bias `bias`,
    `mbits` mantissa bits; `max` its largest finite magnitude and `emax`
    floor(log2(max)), the exponent the block scale is taken against."""

    def __init__(self, name, ebits, mbits, bias, vmax, nan_code=None):
        self.name, self.ebits, self.mbits, self.bias = name, ebits, mbits, bias
        self.max = vmax
        self.emax = int(np.floor(np.log2(vmax)))
        self.emin = 1 - bias                      # exponent of the smallest normal
        self.nan_code = nan_code                  # low bits of the NaN code (E4M3 only)
        self.ncodes = 1 << (1 + ebits + mbits)
        self.table = self._values(np.arange(self.ncodes))

    def _values(self, code):
        """Value of each code from its bit fields (fp64)."""
        c = np.asarray(code, dtype=np.int64)
        m = self.mbits
        sign = np.where((c >> (self.ebits + m)) & 1, -1.0, 1.0)
        ef = (c >> m) & ((1 << self.ebits) - 1)
        mf = c & ((1 << m) - 1)
        mag = np.where(ef == 0, np.ldexp(mf.astype(np.float64), self.emin - m),
                       np.ldexp(((1 << m) + mf).astype(np.float64), ef - 1 + self.emin - m))
        if self.nan_code is not None:
            low = c & ((1 << (self.ebits + m)) - 1)
            mag = np.where(low == self.nan_code, np.nan, mag)
        return sign * mag

    def encode(self, v) -> np.ndarray:
        """Codes of values with |v| <= max, nearest, ties to even: as
        e4m3_encode, with the binade exponent floored at emin and the code's
        magnitude bits 2^m (e - emin) + q."""
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        if np.any(a > self.max) or np.any(np.isnan(a)):
            raise ValueError(f"{self.name}: value outside [-{self.max}, {self.max}]")
        m = self.mbits
        _, ex = np.frexp(np.maximum(a, 2.0 ** (self.emin - 1)))
        e = np.maximum(ex.astype(np.int64) - 1, self.emin)
        q = np.rint(np.ldexp(a, m - e)).astype(np.int64)
        code = (1 << m) * (e - self.emin) + q
        code |= (v < 0).astype(np.int64) << (self.ebits + m)
        return code.astype(np.uint8)

    def decode(self, code) -> np.ndarray:
        return self.table[np.asarray(code, dtype=np.uint8)]


FORMATS = {
    "e4m3": ElementFormat("e4m3", 4, 3, 7, 448.0, nan_code=0x7F),
    "e2m3": ElementFormat("e2m3", 2, 3, 1, 7.5),
    "e3m2": ElementFormat("e3m2", 3, 2, 3, 28.0),
    "e2m1": ElementFormat("e2m1", 2, 1, 1, 6.0),
}


def e8m0_decode(code) -> np.ndarray:
    """2^(code - 127) as fp64 (code 255, the NaN code, is never produced)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    return np.ldexp(1.0, c - 127)


def mx_quantize(v, axis: int = -1, fmt: str = "e4m3"):
    """Quantise ``v`` in blocks of 32 along ``axis`` to element format ``fmt``
    (E4M3 by default) with one E8M0 scale per block.

    Returns (codes uint8, same shape as v; scales uint8, that axis divided by 32).
    """
    F = FORMATS[fmt]
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError(f"mx_quantize: axis length {n} is not a multiple of {BLOCK}")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.max(np.abs(b), axis=-1)
    _, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 1                 # floor(log2 amax) for amax > 0
    s = np.clip(e - F.emax, -127, 127)
    s = np.where(amax == 0, -127, s)
    scaled = np.clip(np.ldexp(b, -s[..., None]), -F.max, F.max)
    enc = e4m3_encode if fmt == "e4m3" else F.encode
    codes = enc(scaled).reshape(v.shape)
    scales = (s + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes, scales, axis: int = -1, fmt: str = "e4m3") -> np.ndarray:
    """Inverse of :func:`mx_quantize` (exact)."""
    c = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    s = np.moveaxis(np.asarray(scales, dtype=np.uint8), axis, -1)
    dec = e4m3_decode if fmt == "e4m3" else FORMATS[fmt].decode
    vals = dec(c).reshape(c.shape[:-1] + (c.shape[-1] // BLOCK, BLOCK))
    out = vals * e8m0_decode(s)[..., None]
    return np.moveaxis(out.reshape(c.shape), -1, axis)


def mx_roundtrip(v, axis: int = -1, fmt: str = "e4m3") -> np.ndarray:
    """deq(MXQ(v)): the value a consumer of the quantised tensor sees."""
    c, s = mx_quantize(v, axis, fmt)
    return mx_dequantize(c, s, axis, fmt)


def mx_rows_roundtrip(v) -> np.ndarray:
    """deq(MXQ(v)) with the 32-value blocks running down the rows (axis 0) of
    a 2-D tensor: rows 32b .. 32b+31 of each column share one scale.  A row
    count that is not a multiple of 32 is zero-padded for the quantisation
    (zeros change no block maximum and quantise to zero); the pad is dropped.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    pad = (-n) % BLOCK
    if pad:
        v = np.concatenate([v, np.zeros((pad,) + v.shape[1:])], axis=0)
    return mx_roundtrip(v, axis=0)[:n]
