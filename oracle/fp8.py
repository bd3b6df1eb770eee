"""FP8 linear layers with tensor-wise scaling -- oracle (test infrastructure only).

[nanochat] "3. precision management": with --fp8 most linear layers become
Float8Linear with tensor-wise scaling; master weights stay fp32.

READINGS (the page names the layer type and the scaling granularity only):
  * formats: the OCP 8-bit floats.  e4m3 ("fn": bias 7, no infinities, max
    448) for activations and weights, e5m2 (bias 15, max 57344) for
    gradients -- the usual FP8 training split.
  * scale (per tensor, dynamic): s = fmax / max(amax, 1e-12) in fp32, amax =
    max |x| over the whole tensor; q = fp8(clamp(fp32(x * s), -fmax, fmax)),
    rounded to nearest, ties to even.
  * product: y = (qa . qb^T) * (1/sa) * (1/sb), the reciprocals taken in
    fp32, accumulation exact here (fp64), the result stored as bf16.
"""
from __future__ import annotations

import numpy as np

from .gpt import round_bf16

# (exponent bits, mantissa bits, bias, largest finite value)
FORMATS = {
    "e4m3": (4, 3, 7, 448.0),
    "e5m2": (5, 2, 15, 57344.0),
}
AMAX_FLOOR = np.float32(1e-12)


def fp8_round(y, fmt: str) -> np.ndarray:
    """Nearest value of the format (ties to even) for finite |y| <= max.

    Inside the binade [2^e, 2^(e+1)) the values are spaced 2^(e - mbits); below
    the smallest normal 2^(1 - bias) the spacing stays 2^(1 - bias - mbits)
    (subnormals).  Dividing by the spacing gives an integer grid, where
    numpy's rint rounds half to even -- the even grid point is the one with
    an even mantissa code."""
    ebits, mbits, bias, fmax = FORMATS[fmt]
    y = np.asarray(y, np.float64)
    if np.any(np.abs(y) > fmax) or not np.all(np.isfinite(y)):
        raise ValueError("fp8_round takes finite values within the format's range")
    _, e2 = np.frexp(y)                       # |y| = f 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, 1 - bias)          # binade exponent, floored at the normals'
    q = np.ldexp(1.0, e - mbits)              # spacing
    return np.where(y == 0, 0.0, np.rint(y / q) * q)


def fp8_encode(v, fmt: str) -> np.ndarray:
    """Bit codes (uint8) of values that are exactly representable."""
    ebits, mbits, bias, _ = FORMATS[fmt]
    v = np.asarray(v, np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    _, e2 = np.frexp(a)
    e = e2 - 1
    normal = (a > 0) & (e >= 1 - bias)
    ef = np.where(normal, e + bias, 0)
    mant = np.where(normal, a / np.ldexp(1.0, np.where(normal, e, 0)) - 1.0,
                    a / np.ldexp(1.0, 1 - bias))
    m = np.rint(mant * (1 << mbits))
    assert np.all(m == mant * (1 << mbits)), "value not representable"
    return (sign | (ef.astype(np.uint8) << mbits) | m.astype(np.uint8)).astype(np.uint8)


def fp8_decode(codes, fmt: str) -> np.ndarray:
    """Values of bit codes, written from the field definitions (NaN codes
    map to NaN, e5m2's infinity codes to +-inf)."""
    ebits, mbits, bias, _ = FORMATS[fmt]
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    ef = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    val = np.where(ef == 0, m / (1 << mbits) * 2.0 ** (1 - bias),
                   (1 + m / (1 << mbits)) * np.exp2(ef - bias))
    if fmt == "e4m3":
        val = np.where((ef == 15) & (m == 7), np.nan, val)
    else:
        val = np.where(ef == 31, np.where(m == 0, np.inf, np.nan), val)
    return s * val


def tensor_scale(x, fmt: str) -> np.float32:
    """s = fmax / max(amax, 1e-12), fp32."""
    amax = np.float32(np.max(np.abs(np.asarray(x, np.float32)))) if np.size(x) else np.float32(0)
    return np.float32(np.float32(FORMATS[fmt][3]) / np.maximum(amax, AMAX_FLOOR))


def quantize(x, fmt: str):
    """(codes, values, s, 1/s) of x cast with its tensor-wise scale."""
    fmax = np.float32(FORMATS[fmt][3])
    s = tensor_scale(x, fmt)
    y = np.clip(np.asarray(x, np.float32) * s, -fmax, fmax)   # fp32 product
    v = fp8_round(y, fmt)
    return fp8_encode(v, fmt), v, s, np.float32(np.float32(1) / s)


def scaled_mm(qa, inv_sa, qb, inv_sb) -> np.ndarray:
    """(qa qb^T) (1/sa) (1/sb) in fp64, qa [M, K], qb [N, K] fp8 values."""
    return (np.asarray(qa, np.float64) @ np.asarray(qb, np.float64).T) \
        * np.float64(inv_sa) * np.float64(inv_sb)


def fp8_linear(x, w, fmt_x: str = "e4m3", fmt_w: str = "e4m3") -> np.ndarray:
    """Float8Linear forward y = x w^T with tensor-wise scales, bf16 out."""
    _, qx, _, ix = quantize(x, fmt_x)
    _, qw, _, iw = quantize(w, fmt_w)
    return round_bf16(scaled_mm(qx, ix, qw, iw).astype(np.float32))
