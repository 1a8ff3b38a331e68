"""Helpers for the GPU parity tests: host <-> device bf16 bit patterns, seeded
cases, and the three-part attention check.

Attention parity ([charlestar] "change A, not B": equality within a float
tolerance, not bitwise) is checked in three parts against the fp64 oracle:
  (i)   the kernel's fp32 output (same schedule, written before the final
        rounding) is within 1e-2 max-abs of the oracle;
  (ii)  the bf16 product output equals the round-to-nearest-even of (i)
        bit for bit;
  (iii) the raw bf16 output's max-abs error is reported, with elements of
        |o| >= 4 (where half a bf16 ulp already exceeds 1e-2) kept apart.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

ATOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def three_part_check(out_f32: torch.Tensor, out_bf16: torch.Tensor, ref: np.ndarray,
                     rows=None, atol: float = ATOL) -> dict:
    """Apply checks (i)-(iii); ``rows`` selects sampled rows of full outputs."""
    f32 = out_f32.detach().cpu().numpy().astype(np.float64)
    b16 = host_bits(out_bf16)
    if rows is not None:
        f32, b16 = f32[rows], b16[rows]
    err_f32 = np.abs(f32 - ref)
    assert np.isfinite(f32).all(), "non-finite fp32 output"
    rne = host_bits(torch.from_numpy(f32.astype(np.float32)).to(torch.bfloat16))
    mism = int((rne != b16).sum())
    raw = np.abs(bf16_bits_to_f64(b16) - ref)
    big = np.abs(ref) >= 4.0
    rep = {
        "max_abs_f32": float(err_f32.max()),
        "bf16_vs_rne_mismatches": mism,
        "max_abs_bf16": float(raw.max()),
        "max_abs_bf16_small": float(raw[~big].max()) if (~big).any() else 0.0,
        "n_abs_ge_4": int(big.sum()),
    }
    say("    parity", rep)
    assert rep["max_abs_f32"] <= atol, rep
    assert mism == 0, rep
    return rep


# ------------------------------------------------------------ gradients

U_BF16 = 2.0 ** -8          # unit roundoff of bf16 (8 significand bits)
U_F32 = 2.0 ** -24
TAU = 2.0 ** -126           # smallest normal fp32: values below it are flushed


U_F16 = 2.0 ** -11          # unit roundoff of fp16 (11 significand bits)
TAU_F16 = 2.0 ** -24        # smallest fp16 subnormal: the absolute error floor of an fp16 rounding


def grad_error_bounds(q, k, v, dout, cu, causal=True, heads=None, segments=None, f16=False):
    """Elementwise first-order bounds on the backward kernels' fp32 gradient error.

    The kernels take the forward's 16-bit output O and its fp32 log-sum-exp,
    recompute P in fp32, round P (for dV) and dS = P o (dP - D) (for dQ, dK)
    to the 16-bit input type, and accumulate in fp32.  Inputs are bf16 bit
    patterns, or fp16 arrays with ``f16``.  With u the unit roundoff of that
    type,
    e = 2u + (n + d) 2^-24 per product term (one rounding of the operand, the
    log-sum-exp's relative error from summing bf16 probabilities, fp32 sums),
    W = P |V| (an upper bound of |O| and of the forward's PV error scale) and
    dD_i = 3u sum_d |dO_id| W_id (bf16 O and the forward's own rounding):
      |d dV_jd| <= e sum_i P_ij |dO_id|
      |d dQ_id| <= s sum_j (e |dS_ij| + P_ij dD_i) |K_jd|
      |d dK_jd| <= s sum_i (e |dS_ij| + P_ij dD_i) |Q_id|
    P and dS here are fp64 values computed from the same 16-bit inputs; second
    order terms are dropped.  fp32 values below 2^-126 are flushed to zero by
    the hardware (exp2, the bf16 conversions, MFMA), so every probability and
    every dS term also carries an absolute error tau = 2^-126 (times
    1 + |dP - D| for dS), and every sum n 2^-126; with fp16 operands tau is
    the fp16 rounding's absolute floor 2^-24 instead (values below fp16's
    normal range keep fewer bits).  With M the visibility mask:
      |d dV_jd| += tau sum_i M_ij |dO_id| + n tau
      |d dQ_id|, |d dK_jd| += s sum tau (1 + |dP_ij - D_i|) M_ij |K_jd| (|Q_id|) + n tau
    Entries outside ``heads`` / ``segments`` are NaN.
    """
    if f16:
        Q, K, V, G = (np.asarray(x, np.float16).astype(np.float64) for x in (q, k, v, dout))
        u, tau = U_F16, TAU_F16
    else:
        Q, K, V, G = (bf16_bits_to_f64(x) for x in (q, k, v, dout))
        u, tau = U_BF16, TAU
    T, H, d = Q.shape
    s = 1.0 / np.sqrt(d)
    cu = np.asarray(cu, np.int64)
    heads = range(H) if heads is None else list(heads)
    segments = range(cu.shape[0] - 1) if segments is None else list(segments)
    bq, bk, bv = (np.full((T, H, d), np.nan) for _ in range(3))
    for r in segments:
        a, b = int(cu[r]), int(cu[r + 1])
        n = b - a
        e = 2 * u + (n + d) * U_F32
        for h in heads:
            q_, k_, v_, g_ = Q[a:b, h], K[a:b, h], V[a:b, h], G[a:b, h]
            S = s * (q_ @ k_.T)
            M = np.tril(np.ones((n, n))) if causal else np.ones((n, n))
            S[M == 0] = -np.inf
            S -= S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            O = P @ v_
            W = P @ np.abs(v_)
            dPD = g_ @ v_.T - (g_ * O).sum(axis=1)[:, None]
            dS = P * dPD
            dD = 3 * u * (np.abs(g_) * W).sum(axis=1)
            E = e * np.abs(dS) + P * dD[:, None] + tau * (1 + np.abs(dPD)) * M
            bv[a:b, h] = (e * P + tau * M).T @ np.abs(g_) + n * TAU
            bq[a:b, h] = s * (E @ np.abs(k_)) + n * TAU
            bk[a:b, h] = s * (E.T @ np.abs(q_)) + n * TAU
    return bq, bk, bv


def grad_check(got_f32, got_bf16, refs, bounds, rows=None) -> dict:
    """fp32 gradients within their elementwise bounds of the fp64 oracle (where
    the oracle was evaluated), and 16-bit gradients (bf16 or fp16) equal to the
    RNE rounding of the fp32 ones bit for bit."""
    rep = {}
    idx = None if rows is None else torch.as_tensor(np.asarray(rows, np.int64), device=got_f32[0].device)
    for name, f, b16, ref, bnd in zip(("dq", "dk", "dv"), got_f32, got_bf16, refs, bounds):
        if idx is not None:       # select on the device: full-size gradients stay there
            f, b16, ref, bnd = f[idx], b16[idx], ref[rows], bnd[rows]
        f = f.detach().cpu().numpy().astype(np.float64)
        bits = host_bits(b16)
        assert np.isfinite(f).all(), f"non-finite {name}"
        sel = np.isfinite(ref)
        err = np.abs(f - ref)[sel]
        lim = bnd[sel]
        rne = host_bits(torch.from_numpy(f.astype(np.float32)).to(b16.dtype))
        rep[name] = {
            "max_abs_err": float(err.max()),
            "max_err_over_bound": float((err / np.maximum(lim, 1e-300)).max()),
            "max_abs_ref": float(np.abs(ref[sel]).max()),
            "rne_mismatches_16bit": int((rne != bits).sum()),
        }
    say("    grad parity", rep)
    for name, r in rep.items():
        assert r["max_err_over_bound"] <= 1.0, (name, r)
        assert r["rne_mismatches_16bit"] == 0, (name, r)
    return rep
