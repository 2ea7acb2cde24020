"""fp8 e4m3 encoding for the low-bit projections.

Source: PaperDaily review, section 2 (Flash): suitable projections use low-bit
weights and activations, with quantisation fused into the normalisation. The
pages give no format or scale rule. Readings:
  * format: OCP e4m3 "fn" (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, no infinities, largest finite 448, subnormal step 2**-9);
  * rounding: to the nearest representable value, ties to the even code;
    magnitudes above 448 saturate to 448;
  * scales: one per tensor. Weights: static s_W = amax(W) / 448, codes of
    W * (448 / amax(W)), both evaluated in IEEE fp32 (the precision the GPU
    quantiser uses, so that both sides produce the same bytes). Activations:
    dynamic s_A = amax(A) / 448 per GEMM input (amax 0 -> scale 1).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _positive_table() -> np.ndarray:
    """Values of codes 0..126 (sign bit clear), ascending with the code."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** -6)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.asarray(vals, dtype=np.float64)


_POS = _positive_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, _POS[np.minimum(c & 0x7F, 126)])
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Finite float array -> uint8 e4m3fn codes: nearest value, ties to even
    code, saturating at +-448, sign kept (so -0.0 and tiny negatives -> 0x80).

    Inside the binade [2^E, 2^(E+1)) (E >= -6; below 2^-6 the subnormal step
    continues the E = -6 grid) the representable values are the multiples of
    2^(E-3); rounding to the nearest multiple with ties to even is np.rint of
    a / 2^(E-3), which is exact in fp64, and the code of k * 2^(E-3) is
    8 (E + 6) + k (a carry to k = 16 lands on the next binade's first code)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode expects finite input")
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)                                   # a = m 2^e, m in [0.5, 1) -> binade E = e - 1
    E = np.where(a < 2.0 ** -6, -6, e - 1)                # zero and subnormals on the E = -6 grid
    k = np.rint(np.ldexp(a, 3 - E))                       # multiples of the grid step 2^(E-3)
    code = (8 * (E + 6) + k).astype(np.int64)
    return (code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def e4m3_encode_nearest(x: np.ndarray) -> np.ndarray:
    """The same map by brute force: the nearest entry of the table of all
    codes (ties to the even code). Slow; used to cross-check e4m3_encode."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_POS, a, side="left"), 126)   # first table value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_POS[hi] == a, hi, code)
    return (code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def quantize_weight_fp8(w: np.ndarray):
    """Per-tensor static weight quantisation in fp32: returns (codes uint8,
    scale float32) with W ~= decode(codes) * scale."""
    w32 = np.ascontiguousarray(w, dtype=np.float32)
    amax = np.float32(np.max(np.abs(w32))) if w32.size else np.float32(0)
    if amax == 0:
        inv, scale = np.float32(1), np.float32(1)
    else:
        inv = np.float32(E4M3_MAX) / amax
        scale = amax / np.float32(E4M3_MAX)
    q = (w32 * inv).astype(np.float32)
    return e4m3_encode(q), np.float32(scale)


def round_to(a: np.ndarray, precision: str) -> np.ndarray:
    """Round fp64 values to the nearest value of `precision` ("f64", "f32" or
    "bf16"; ties to even), returned as fp64. bf16 keeps the top 16 bits of
    the fp32 pattern: round-half-even on the 16 dropped bits of the fp32
    value (finite inputs only)."""
    a = np.asarray(a, dtype=np.float64)
    if precision == "f64":
        return a
    a32 = a.astype(np.float32)
    if precision == "f32":
        return a32.astype(np.float64)
    if precision != "bf16":
        raise ValueError(precision)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_act_fp8(a: np.ndarray, precision: str = "f64"):
    """Per-tensor dynamic activation quantisation: returns (decoded e4m3
    values, scale s) with a ~= values * s. This is what the low-bit GEMM
    consumes: (values @ W_codes^T) * s * s_W.

    A code is an integer decided by floating point, so it is decided in the
    precision the quantised tensor is held in (`precision`): the values are
    first rounded to it, amax is taken over the rounded values, and with
    "f32" or "bf16" the scaled value a * (448 / amax) is formed in IEEE fp32
    (the factor itself correctly rounded to fp32) before the e4m3 rounding.
    "f64" does all of it in fp64."""
    a = round_to(a, precision)
    amax = float(np.max(np.abs(a))) if a.size else 0.0
    s = amax / E4M3_MAX if amax > 0 else 1.0
    if precision == "f64":
        scaled = a / s
    else:
        inv = np.float32(E4M3_MAX) / np.float32(amax) if amax > 0 else np.float32(1)
        scaled = (a.astype(np.float32) * inv).astype(np.float64)
    return e4m3_decode(e4m3_encode(scaled)), s
