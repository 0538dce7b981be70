"""NVFP4 quantizer, dequantizer and FP64 linear: the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, written
for a reader who checks it against the definitions by eye; nothing is blocked,
fused or reordered.

Where the pages leave a step open, the plainest reading is taken:

* Format (the pages name "NVFP4 (W4A4)" -- README, intro paragraph and
  "Supported models"; arXiv abstract "hardware-supported low-precision
  execution"): value = e2m1(code) * e4m3(block scale) * fp32(tensor scale),
  blocks of 16 consecutive elements along K, the reduction axis, for both the
  weight rows and the activation rows, so that block j of an activation row
  meets block j of a weight row.
* Tensor scale: s_g = amax / (6 * 448) in binary32, so that the tensor's
  largest magnitude maps onto the largest E2M1 magnitude (6) times the largest
  E4M3 scale (448).  amax == 0 gives s_g = 1.
* Operation order (decides rounding ties, therefore bit-exactness): per block
  sigma = a / (s_g * 6); scale byte = E4M3 round-to-nearest-even of sigma,
  saturating at 448; T = S * s_g; r = 1 / T (0 when T == 0); y = x * r;
  element code = E2M1 round-to-nearest-even of |y|, saturating at 6, with the
  sign bit taken from the sign of x (so -0 and negative underflow give 0x8).
  Every step is one IEEE binary32 operation with round-to-nearest-even and no
  fused multiply-add.
* Canonical layout: codes [R][K/2] with element 2i in bits 0..3 and element
  2i+1 in bits 4..7 of byte i; scales [R][K/16]; one binary32 tensor scale.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
_F32 = np.float32


# --------------------------------------------------------------------------
# Element formats
# --------------------------------------------------------------------------

def e2m1_decode(code) -> np.ndarray:
    """Value of 4-bit E2M1 codes, float64.

    OCP MX v1.0, section 5.3.3: 1 sign bit, 2 exponent bits (bias 1), 1
    mantissa bit, subnormal when the exponent field is 0, no Inf or NaN.
    value = (-1)^s * (e == 0 ? 0.5*m : 2^(e-1) * (1 + m/2)).
    Pinned by tests/golden/e2m1_values.txt (the spec's value table).
    """
    c = np.asarray(code, dtype=np.int64) & 0xF
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e4m3_decode(byte) -> np.ndarray:
    """Value of E4M3 ("FN") bytes, float64; NaN for 0x7F / 0xFF.

    OCP OFP8 v1.0: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
    subnormal when the exponent field is 0, no infinities, S.1111.111 is NaN.
    value = (-1)^s * (e == 0 ? m * 2^-9 : 2^(e-7) * (1 + m/8)).
    Pinned exhaustively against torch's float8_e4m3fn -> float32 cast and
    the spec's landmark values (tests/golden/e4m3_landmarks.txt).
    """
    b = np.asarray(byte, dtype=np.int64) & 0xFF
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _nearest_even(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value to each v (v >= 0, grid ascending,
    v <= grid[-1]); a tie between two neighbours goes to the even index.

    The comparison is against the exact midpoint of the two neighbours (grid
    values are dyadic rationals with few bits, so their float64 midpoint is
    exact, and every binary32 v is exact in float64).
    """
    v = np.asarray(v, dtype=np.float64)
    hi = np.searchsorted(grid, v, side="left")          # grid[hi-1] < v <= grid[hi]
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    mid = 0.5 * (grid[lo] + grid[hi])
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(v == grid[hi], hi, idx)


_E2M1_GRID = e2m1_decode(np.arange(8))        # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_GRID = e4m3_decode(np.arange(0x7F))     # bytes 0x00 .. 0x7E, ascending


def e2m1_encode(y) -> np.ndarray:
    """E2M1 code of binary32 values y: round |y| to the nearest E2M1
    magnitude, ties to the even code, saturating at 6; the sign bit is the
    sign bit of y (IEEE-style conversion, so -0.0 -> 0x8).

    Pinned by the threshold table, a dense sweep against an independent
    formula and brute force (tests/test_oracle_formats.py).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), E2M1_MAX)
    code = _nearest_even(a, _E2M1_GRID).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def e4m3_encode(sigma) -> np.ndarray:
    """E4M3 byte of non-negative binary32 scale values: nearest E4M3 value,
    ties to the even mantissa (= even byte), saturating at 448 (0x7E).

    Pinned by torch's float8_e4m3fn cast over every binary32 value in
    [2^-12, 448], the tie table and brute force.
    """
    s = np.asarray(sigma, dtype=np.float32)
    if np.any(s < 0) or np.any(~np.isfinite(s)):
        raise ValueError("block scales are finite and non-negative")
    a = np.minimum(s.astype(np.float64), E4M3_MAX)
    return _nearest_even(a, _E4M3_GRID).astype(np.uint8)


# --------------------------------------------------------------------------
# Nibble packing (canonical layout)
# --------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R][K] 4-bit codes -> [R][K/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[R][K/2] bytes -> [R][K] 4-bit codes (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------

@dataclass
class NVFP4Tensor:
    """Canonical NVFP4 tensor: codes [R][K/2], scales [R][K/16] (uint8) and
    the binary32 tensor scale (a 0-d float32, or [R] when per_row)."""
    codes: np.ndarray
    scales: np.ndarray
    gscale: np.ndarray

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def global_scale(x: np.ndarray) -> tuple[np.float32, np.float32]:
    """(amax, s_g) of a binary32 tensor: amax = max |x| (exact);
    s_g = amax / 2688 in binary32, replaced by 1 when it is 0."""
    x = np.asarray(x, dtype=np.float32)
    amax = _F32(np.max(np.abs(x))) if x.size else _F32(0.0)
    sg = _F32(amax / _F32(E2M1_MAX * E4M3_MAX))
    if sg == _F32(0.0):
        sg = _F32(1.0)
    return amax, sg


def quantize_blocks(x: np.ndarray, sg) -> tuple[np.ndarray, np.ndarray]:
    """Block scales and element codes of x [R][K] (K % 16 == 0) given the
    tensor scale s_g; returns (codes [R][K/2], scales [R][K/16]).

    Steps, each a binary32 operation:
      a     = max |x_i| over the 16-element block
      d     = s_g * 6
      sigma = a / d
      b     = e4m3_encode(sigma);  S = e4m3_decode(b)
      T     = S * s_g
      r     = 0 if T == 0 else 1 / T
      y_i   = x_i * r
      c_i   = e2m1_encode(y_i)   (sign from x_i)
    """
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    sg = _F32(sg)
    xb = x.reshape(R, K // BLOCK, BLOCK)
    a = np.max(np.abs(xb), axis=2)                           # [R][K/16] f32
    d = _F32(sg * _F32(E2M1_MAX))
    sigma = (a / d).astype(np.float32)
    b = e4m3_encode(sigma)
    S = e4m3_decode(b).astype(np.float32)
    T = (S * sg).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(T == 0, _F32(0.0), _F32(1.0) / T).astype(np.float32)
    y = (xb * r[:, :, None]).astype(np.float32)
    codes = e2m1_encode(y).reshape(R, K)
    return pack_nibbles(codes), b


def quantize(x: np.ndarray, per_row: bool = False) -> NVFP4Tensor:
    """NVFP4-quantize a binary32 (typically bf16-valued) tensor [R][K].

    per_row=False (the path's reading): one tensor scale over the whole R x K
    tensor.  per_row=True: every row is quantized as its own tensor.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize expects a 2-D [R][K] array")
    if per_row:
        codes = np.empty((x.shape[0], x.shape[1] // 2), np.uint8)
        scales = np.empty((x.shape[0], x.shape[1] // BLOCK), np.uint8)
        gs = np.empty(x.shape[0], np.float32)
        for i in range(x.shape[0]):
            _, gs[i] = global_scale(x[i:i + 1])
            codes[i:i + 1], scales[i:i + 1] = quantize_blocks(x[i:i + 1], gs[i])
        return NVFP4Tensor(codes, scales, gs)
    _, sg = global_scale(x)
    codes, scales = quantize_blocks(x, sg)
    return NVFP4Tensor(codes, scales, np.asarray(sg, dtype=np.float32))


def dequantize(q: NVFP4Tensor) -> np.ndarray:
    """x_hat = e2m1(code) * e4m3(scale) * s_g in float64 (exact: at most
    2 + 4 + 24 significant bits)."""
    c = e2m1_decode(unpack_nibbles(q.codes))
    S = np.repeat(e4m3_decode(q.scales), BLOCK, axis=1)
    g = np.asarray(q.gscale, dtype=np.float64)
    if g.ndim == 1:
        g = g[:, None]
    return c * S * g


# --------------------------------------------------------------------------
# Linear
# --------------------------------------------------------------------------

def linear_ref(xq: NVFP4Tensor, wq: NVFP4Tensor) -> np.ndarray:
    """y[m, n] = sum_k x_hat[m, k] * w_hat[n, k] in float64 (one BLAS matmul
    of the dequantized operands; relative error <= K * 2^-53)."""
    return dequantize(xq) @ dequantize(wq).T


def linear_exact(xq: NVFP4Tensor, wq: NVFP4Tensor):
    """The same sum in exact rational arithmetic (every x_hat and w_hat is a
    dyadic rational).  Tiny shapes only; returns a nested list of Fraction."""
    xh = dequantize(xq)
    wh = dequantize(wq)
    X = [[Fraction(float(v)) for v in row] for row in xh]
    W = [[Fraction(float(v)) for v in row] for row in wh]
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in W] for xr in X]


def tolerance_bound(xq: NVFP4Tensor, wq: NVFP4Tensor, rel: float = 1e-3) -> np.ndarray:
    """Per-element bound rel * sum_k |x_hat[m,k] * w_hat[n,k]| (float64).

    Pinned by exact rational sums built from the spec value tables under
    tests/golden/ with distinct block and tensor scales (rel = 1 and the
    default rel = 1e-3), and by a cancelling dot whose output is 0 while the
    bound is not (tests/test_oracle_dot.py)."""
    return rel * (np.abs(dequantize(xq)) @ np.abs(dequantize(wq)).T)
