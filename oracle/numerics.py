"""Plain fp64 building blocks of the decoder (ORACLE — test infrastructure only).

Each function is the textbook definition, evaluated in float64 with numpy.
The rounding points of the storage contract (bf16 at GEMM inputs, bf16 q/k/v,
fp32 residual) are applied by the callers in ``oracle/model.py`` through
``round_act``.
"""
from __future__ import annotations

import numpy as np

SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 keeps 8 significant bits and fp32's exponent range; the
    quantum is 2^(e-8) for x = m*2^e, m in [0.5, 1), and 2^-133 in the
    subnormal range."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(x / q) * q


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps), gain 1 (no learned gain in the synthetic models)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation (Hendrycks & Gimpel, 2016, section 2)."""
    return 0.5 * x * (1.0 + np.tanh(SQRT_2_OVER_PI * (x + 0.044715 * x ** 3)))


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding (Su et al., RoFormer, 2021, section 3.4.2):
    each pair (2j, 2j+1) of a head vector at position p is rotated by the angle
    p * base^(-2j/d).  x: [..., T, H, d]; positions: [T]."""
    d = x.shape[-1]
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]  # [T, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def softmax(a: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(a, axis=axis, keepdims=True)
    e = np.exp(a - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def entropy_direct(p: np.ndarray) -> np.ndarray:
    """H = -sum p ln p with 0 ln 0 = 0, per row."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0.0, p * np.log(np.where(p > 0.0, p, 1.0)), 0.0)
    return -np.sum(t, axis=-1)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round to the OCP FP8 E4M3 grid (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, max finite 448, no infinities), ties to even; values
    beyond 448 saturate.  Returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5,1)
    # normal quantum 2^(e-4) (4 significant bits); subnormal quantum 2^-9
    q = np.ldexp(1.0, np.maximum(e - 4, -9))
    r = np.rint(a / q) * q
    r = np.minimum(r, 448.0)
    return np.sign(x) * r


def e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code (OCP 8-bit floating point specification,
    E4M3 encoding): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN and
    there are no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of an array of E4M3 codes (the 256 values of e4m3_value)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_value(code: int) -> float:
    """Value of one FP4 E2M1 element code (OCP Microscaling Formats v1.0, the
    FP4 element type): sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
    exponent field 0 holds the subnormal m/2; no infinities or NaN."""
    sign = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 0x3, code & 0x1
    if e == 0:
        return sign * (m / 2.0)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """float64 values of an array of E2M1 codes (one code per byte, 0..15)."""
    c = np.asarray(codes, dtype=np.uint8)
    if np.any(c > 15):
        raise ValueError("E2M1 codes are 4-bit")
    return _E2M1_TABLE[c]


def e8m0_decode(codes) -> np.ndarray:
    """float64 values of E8M0 scale codes (OCP Microscaling Formats v1.0, the
    shared scale): 2^(code - 127), code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def mxfp4_dequantize(codes, scales) -> np.ndarray:
    """The values of an MXFP4 tensor [rows][cols]: element code (r, c) times
    the scale of its block of 32, (r, c / 32), exactly in float64."""
    codes = np.asarray(codes)
    sc = e8m0_decode(scales)
    return e2m1_decode(codes) * np.repeat(sc, 32, axis=-1)
