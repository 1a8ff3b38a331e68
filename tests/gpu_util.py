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
