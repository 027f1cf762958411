"""ORACLE (test infrastructure only): number formats, written from their definitions.

* bf16: 1 sign, 8 exponent, 7 stored mantissa bits (IEEE-754 binary32 truncated to its top 16
  bits); rounding is round-to-nearest, ties-to-even (RNE). The model and its compute precision are
  bf16 [youdonthavefriends cost analysis, "config appendix": dtype bf16, precision bf16].
* e4m3fn (OCP FP8 E4M3): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; 0x7F/0xFF
  are NaN; largest finite 448 = 1.75 * 2^8; subnormals k * 2^-9 (k = 1..7).
* dynamic tensorwise quantisation, the scaling of the FP8 GEMMs
  [hn.213312.xyz translation, "提升吞吐量 / Increasing throughput": FP8 with dynamic scaling on
  three GEMMs; linlog.top article, "吞吐量优化": torch._scaled_mm with dynamic tensorwise scales].
  The pages name the scheme, not its constants; the constants below are the reading taken:
    amax      = max |x| over the whole tensor
    ratio     = fl32(448 / max(amax, fl32(1e-12)))     (IEEE fp32 division)
    scale     = 2^floor(log2(ratio))                   (the largest power of two <= ratio)
    q         = e4m3_RNE(clamp(fl32(x * scale), -448, 448))
    inv_scale = 1 / scale                              (exact)
  and a GEMM of quantised operands is dequantised as (sum of exact products) * inv_a * inv_b.
  A power-of-two scale makes x * scale exact and keeps the scale unchanged when amax moves by a
  rounding error (it changes only when amax crosses a power of two); an unrounded 448 / amax
  would re-grid every element of the tensor whenever its single largest element changes by one
  bf16 ulp.
  This departs from the plainest reading, scale = fl32(448 / amax) with no rounding (the default
  of the torch._scaled_mm tensorwise recipes). It was adopted after measurement, for a reason of
  comparability, not of accuracy: with the unrounded ratio a GPU path and this oracle, which agree
  up to fp32-vs-float64 rounding upstream, pick scales one ulp apart whenever the largest element
  of relu(u)^2 differs by one bf16 ulp, and the FP8 MLP outputs then drift ~3% apart (beyond a
  2e-2 parity bar); with a power of two they pick the same scale except when amax lies within
  rounding of a binade edge. Both readings quantise to 4 significant bits; the power of two uses
  between half and all of the e4m3 range (largest code 224..448) instead of all of it.
  Pins: a scale found by search over powers of two (tests/torch_fp8.py) and torch's own e4m3 cast;
  the FP8 GEMMs of oracle.model against torch._scaled_mm compositions, with planted mistakes.

All arithmetic is float64; a float64 result of one fp32 op on fp32 operands, rounded once to
fp32, is the correctly rounded fp32 result (53 >= 2*24 + 2), so the fp32 steps above are exact.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6      # smallest normal: 2^-6
E4M3_MANT_BITS = 3
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9
AMAX_FLOOR = float(np.float32(1e-12))


def f32(x):
    """Round float64 values to the nearest float32 (RNE) and return them as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round each value of x (float64, finite, |x| < 2^128) to the nearest bf16, ties to even.

    A nonzero x = m * 2^e with 0.5 <= |m| < 1 has 8 significant bits in bf16, so its quantum is
    2^(e-8); below the smallest normal 2^-126 the quantum is fixed at 2^-133 (subnormals).
    x / quantum is exact in float64 and numpy's rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)               # |x| < 2^-126  ->  quantum 2^-133
    quantum = np.ldexp(1.0, e - 8)
    return np.rint(x / quantum) * quantum


def bf16_bits_of(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are already bf16-representable."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# e4m3fn
# ----------------------------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3fn code (uint8) as float64; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = m * E4M3_SUBNORMAL_QUANTUM
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_round(v) -> np.ndarray:
    """Round finite values with |v| <= 448 to the nearest e4m3fn value, ties to even.

    For |v| >= 2^-6, |v| = m * 2^e (0.5 <= m < 1) has 4 significant bits, quantum 2^(e-4);
    below 2^-6 the quantum is the subnormal step 2^-9. Signed zero is kept (np.rint keeps it).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3_round expects finite values clamped to [-448, 448]")
    _, e = np.frexp(v)
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP + 1)   # below 2^-6: quantum 2^(-5-4) = 2^-9
    quantum = np.ldexp(1.0, e - (E4M3_MANT_BITS + 1))
    return np.rint(v / quantum) * quantum


def e4m3_encode(v) -> np.ndarray:
    """Codes (uint8) of values that are exactly e4m3fn-representable (e.g. from e4m3_round)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    _, e = np.frexp(a)
    unb = e - 1                                     # floor(log2 a) for a > 0
    is_norm = a >= 2.0 ** E4M3_MIN_NORMAL_EXP
    exp_field = np.where(is_norm, unb + 7, 0)
    mant_norm = np.rint((a / np.ldexp(1.0, np.where(is_norm, unb, 0)) - 1.0) * 8.0)
    mant_sub = np.rint(a / E4M3_SUBNORMAL_QUANTUM)
    mant = np.where(is_norm, mant_norm, mant_sub).astype(np.int64)
    codes = sign | (exp_field.astype(np.int64) << 3) | mant
    if not np.array_equal(e4m3_decode(codes), v):
        raise ValueError("e4m3_encode: value not representable")
    return codes.astype(np.uint8)


def quantize_tensorwise(x):
    """Dynamic tensorwise e4m3 quantisation of a tensor of fp32/bf16 values (module docstring).

    Returns (codes uint8 same shape, values float64 same shape, scale, inv_scale) where
    values = decode(codes) and scale/inv_scale are float32-representable float64 scalars.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    ratio = float(f32(E4M3_MAX / max(amax, AMAX_FLOOR)))
    _, e = np.frexp(ratio)                        # ratio = m * 2^e, 0.5 <= m < 1
    scale = float(np.ldexp(1.0, int(e) - 1))
    inv_scale = float(np.ldexp(1.0, 1 - int(e)))
    y = f32(x * scale)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    vals = e4m3_round(y)
    codes = e4m3_encode(vals)
    return codes, vals, scale, inv_scale


def fp8_matmul_nt(a_vals, a_inv, b_vals, b_inv):
    """deq(A8 . B8^T): exact products of e4m3 values summed (float64), times inv_a, times inv_b."""
    return (np.asarray(a_vals) @ np.asarray(b_vals).T) * a_inv * b_inv
