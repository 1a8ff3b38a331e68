"""Oracle for rotary position embedding with positions reset per segment.

Test infrastructure only (see the package docstring).

Positions: token i of segment r sits at p_i = i - cu_r ([charlestar] "nine
tokens, three identities"), so every segment starts again from 0 ([vllbc] the
THD RoPE recovers local positions from cu_seqlens; [compass] "cross-
contamination": position ids reset at each segment; [opworld] "pitfall two":
reset positions per document).

Rotation (a reading; the pages fix no RoPE variant): the rotate-half pairing
of a head vector x of width d, pair j < d/2 is (x_j, x_{j+d/2}), turned by the
angle theta_j = p * f_j with f_j = base^(-2j/d):
    y_j       = x_j cos theta - x_{j+d/2} sin theta
    y_{j+d/2} = x_{j+d/2} cos theta + x_j sin theta
Precision contract shared with the device library:
  f_j     computed in double, rounded once to fp32;
  theta_j the fp32 product fp32(p) * f_j (one rounding), so both sides hold the
          same angle bit for bit;
  cos, sin and the rotation in double, then one rounding to bf16 (nearest,
          ties to even).
Interleaved pairing (the RoFormer construction [charlestar] "positions and
RoPE" cites; a flag on the device side): pair j is (x_{2j}, x_{2j+1}), with the
same angle theta_j and the same precision contract:
    y_{2j}   = x_{2j} cos theta - x_{2j+1} sin theta
    y_{2j+1} = x_{2j+1} cos theta + x_{2j} sin theta
The pages' shift-invariance identity ([charlestar] "positions and RoPE"):
(R(m+c)q)^T (R(n+c)k) = q^T R(n-m) k, so a common per-segment offset cancels.
"""

from __future__ import annotations

import math

import numpy as np

from .pack import positions_from_cu


def rope_freqs(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """fp32 [d/2]: f_j = base^(-2j/d), evaluated with libm pow in double."""
    return np.asarray([math.pow(float(base), -2.0 * j / head_dim)
                       for j in range(head_dim // 2)], np.float64).astype(np.float32)


def rope_angles(positions, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """fp32 [n, d/2]: theta = fp32(p) * f_j, one correctly rounded fp32 product."""
    p = np.asarray(positions).astype(np.float32)
    return p[:, None] * rope_freqs(head_dim, base)[None, :]


def bf16_bits_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round doubles straight to bf16 (8 significant bits), nearest, ties to even.

    The mantissa is rounded in the double's own bit pattern, so there is no
    intermediate fp32 rounding.  Assumes normal bf16 results (no subnormals,
    no overflow), which holds for the N(0,1)-scale values used here.
    """
    b = np.ascontiguousarray(x, np.float64).view(np.uint64)
    drop = np.uint64(45)                                  # 52 - 7 mantissa bits
    lsb = (b >> drop) & np.uint64(1)
    half = (np.uint64(1) << np.uint64(44)) - np.uint64(1)
    r = (b + half + lsb) & ~((np.uint64(1) << drop) - np.uint64(1))
    f = r.view(np.float64).astype(np.float32)             # exact: at most 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(x) -> np.ndarray:
    """Round doubles straight to fp16 (11 significant bits, subnormals kept),
    nearest, ties to even: numpy's double-to-half conversion rounds from the
    double's own bits (checked against exact rationals by the tests)."""
    return np.ascontiguousarray(x, np.float64).astype(np.float16).view(np.uint16)


def rotate_f64(x: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Rotate-half rotation in double. x [n, H, d] doubles, theta [n, d/2] fp32 angles."""
    half = x.shape[-1] // 2
    c = np.cos(theta.astype(np.float64))[:, None, :]
    s = np.sin(theta.astype(np.float64))[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rotate_interleaved_f64(x: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Interleaved rotation in double: pair j is (x_{2j}, x_{2j+1})."""
    c = np.cos(theta.astype(np.float64))[:, None, :]
    s = np.sin(theta.astype(np.float64))[:, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


def rope_apply(x_bits: np.ndarray, cu, base: float = 10000.0, rows=None, interleaved: bool = False,
               f16: bool = False) -> np.ndarray:
    """bf16 (or fp16 with ``f16``) bits [T, H, d] -> rotated bits of the same
    type; ``rows`` restricts to those tokens."""
    pos = positions_from_cu(cu)
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        pos, x_bits = pos[rows], x_bits[rows]
    theta = rope_angles(pos, x_bits.shape[-1], base)
    rot = rotate_interleaved_f64 if interleaved else rotate_f64
    if f16:
        return f64_to_f16_bits(rot(f16_bits_to_f64(x_bits), theta))
    return f64_to_bf16_bits(rot(bf16_bits_to_f64(x_bits), theta))
