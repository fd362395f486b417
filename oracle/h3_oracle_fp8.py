"""Plain fp64 CPU oracle for the quantized-score attention variant.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
never calls it and shares no code with it.

The variant: the pages' GB10 correctness baseline for H3 attention is a
quantized attention (SageAttention2, "H3 Parity Evidence Ledger", "Reference
Runs And Immutable Artifacts" and "Completed Findings" tables), and the h3-metal
README ("Implementation and performance notes") reports that quantized attention
changes fine detail.  The "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 4
("Numerical contract"), allows casts only at declared boundaries, so the cast
is declared here as the definition of the variant:

  q8 = e4m3(4 q'),   q' = q_scale * RoPE(RMSNorm(q, gamma_q))
  k8 = e4m3(k' / 4), k' = RoPE(RMSNorm(k, gamma_k))
  s  = q8 k8^T                                   (exact)
  out_i = sum_j 2^(s_ij) v_j / sum_j 2^(s_ij)    (base-2 softmax)

with q_scale = scale * log2(e), so that without the casts this is exactly the
path's softmax(q' k'^T scale) v (the oracle of h3_oracle.py).  The factors 4 and
1/4 are powers of two: they only move both operands into the format's normal
range and cancel in the product.

e4m3 is the OCP 8-bit floating point format E4M3 (OCP "8-bit Floating Point
Specification (OFP8)", revision 1.0): 1 sign, 4 exponent (bias 7) and 3 mantissa
bits, subnormals, no infinities, the one NaN pattern S.1111.111 per sign, largest
finite value 448.  Conversion rounds to nearest, ties to even.  Values that would
round past 448 are outside the variant's domain (its precondition) and raise.

Readings: the prologue outputs are taken exactly (fp64) before the cast; the cast
is the only rounding in the definition.  Pinned by tests/test_oracle_fp8_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

from .h3_oracle import RMS_EPS, mm_rope, rms_norm

E4M3_MAX = 448.0
E4M3_BIAS = 7
E4M3_MIN_NORMAL_EXP = -6   # 2^-6, the smallest normal magnitude
E4M3_MANT_BITS = 3
Q_FACTOR = 4.0             # q' times 4, k' divided by 4


def e4m3_encode(x) -> np.ndarray:
    """float64 -> uint8 e4m3 codes, round to nearest, ties to even.

    A magnitude m with 2^e <= m < 2^(e+1), e >= -6, is a normal number with
    quantum 2^(e-3); below 2^-6 the quantum is fixed at 2^-9 (subnormals).  The
    magnitude is divided by its quantum (exact: a power of two), rounded half to
    even to an integer n, and packed: normal n in [8, 16) -> exponent field
    e + 7 and mantissa n - 8 (n = 16 carries into the next binade); subnormal
    n in [0, 8] -> the code n itself (n = 8 is the smallest normal, code 8).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3_encode: magnitude above 448, outside the format's finite range")
    _, e2 = np.frexp(a)              # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, E4M3_MIN_NORMAL_EXP)  # binade exponent, floor at the normal minimum
    e = np.where(a == 0, E4M3_MIN_NORMAL_EXP, e)
    quantum = np.ldexp(1.0, (e - E4M3_MANT_BITS).astype(np.int32))
    n = np.rint(a / quantum).astype(np.int64)  # numpy rint: half to even
    normal = a >= 2.0 ** E4M3_MIN_NORMAL_EXP
    carry = normal & (n == 16)
    n = np.where(carry, 8, n)
    e = np.where(carry, e + 1, e)
    mag = np.where(normal, ((e + E4M3_BIAS) << E4M3_MANT_BITS) | (n - 8), n)
    if np.any(mag > 0x7E):
        raise ValueError("e4m3_encode: rounds above 448")
    sign = np.signbit(x).astype(np.int64) << 7
    return (sign | mag).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (NaN for the NaN patterns)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> E4M3_MANT_BITS) & 0xF
    m = c & 0x7
    val = np.where(ef == 0, m / 8.0 * 2.0 ** E4M3_MIN_NORMAL_EXP,
                   np.ldexp(1.0 + m / 8.0, (ef - E4M3_BIAS).astype(np.int32)))
    val = np.where((ef == 0xF) & (m == 0x7), np.nan, val)
    return s * val


def e4m3_round(x) -> np.ndarray:
    """x rounded to the nearest e4m3 value (ties to even), as float64."""
    return e4m3_decode(e4m3_encode(x))


def quantized_operands(qr: np.ndarray, kr: np.ndarray, q_scale: float):
    """(q8, k8) values of the prologue outputs qr, kr: e4m3(4 q_scale qr), e4m3(kr / 4)."""
    return (e4m3_round(Q_FACTOR * q_scale * np.asarray(qr, dtype=np.float64)),
            e4m3_round(np.asarray(kr, dtype=np.float64) / Q_FACTOR))


def base2_softmax_rows(s: np.ndarray) -> np.ndarray:
    """2^s_j / sum_j 2^s_j along the last axis (the row maximum subtracted first)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp2(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def quantized_attention_head(q8: np.ndarray, k8: np.ndarray, vh: np.ndarray, block: int = 1024) -> np.ndarray:
    """base-2 softmax(q8 k8^T) vh for one head; q8 [Lq, D], k8/vh [L, D] float64."""
    q8 = np.asarray(q8, dtype=np.float64)
    k8 = np.asarray(k8, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    out = np.empty((q8.shape[0], vh.shape[1]), dtype=np.float64)
    for r0 in range(0, q8.shape[0], block):
        out[r0:r0 + block] = base2_softmax_rows(q8[r0:r0 + block] @ k8.T) @ vh
    return out


def packed_attention_fp8(q, k, v, gamma_q, gamma_k, pos, q_scale: float, eps: float = RMS_EPS) -> np.ndarray:
    """The quantized-score path over [L, H, 128] inputs -> [L, H, 128] float64."""
    qr = mm_rope(rms_norm(np.asarray(q, dtype=np.float64), gamma_q, eps), pos)
    kr = mm_rope(rms_norm(np.asarray(k, dtype=np.float64), gamma_k, eps), pos)
    q8, k8 = quantized_operands(qr, kr, q_scale)
    L, H, D = qr.shape
    out = np.empty((L, H, D), dtype=np.float64)
    for h in range(H):
        out[:, h] = quantized_attention_head(q8[:, h], k8[:, h], np.asarray(v, dtype=np.float64)[:, h])
    return out


def log2e_scale(scale: float) -> float:
    """q_scale for softmax scale `scale`: scale * log2(e), in float64."""
    return scale * math.log2(math.e)
