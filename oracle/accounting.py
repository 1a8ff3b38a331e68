"""Work and waste accounting of packed versus padded layouts.

Test infrastructure only (see the package docstring).  Each helper is the
plain count its page defines:

  [vllbc] "padding waste" equation: waste = (N L - sum l) / (N L) = 1 - mean(l)/L.
  [vllbc] "worked example A" and Table 4-1: fixed slots N L, packs = ceil(T / L)
      (a lower bound), packed slots, saved slots; the table's "score elements"
      column equals sum l^2 / 2 (its label says strict lower triangle, but the
      printed numbers are half the squares; kept here as the page's convention).
  [compass] "intuition" equation: eta = sum L_i / (B L_max).
  [m020] "02 length grouping" and "03": slot totals and sum of squared lengths.
  [charlestar] "two ledgers": padded dense score slots B L_max^2, per-segment
      sum L_r^2, whole-pack T^2, and causal pair counts (19 for [3,2,4]: the
      diagonal is included).
"""

from __future__ import annotations

import math


def waste(lengths, L: int) -> float:
    N = len(lengths)
    return (N * L - sum(lengths)) / (N * L)


def eta(lengths, L_max: int | None = None) -> float:
    L_max = max(lengths) if L_max is None else L_max
    return sum(lengths) / (len(lengths) * L_max)


def packs_lower_bound(lengths, L: int) -> int:
    return math.ceil(sum(lengths) / L)


def table_4_1_row(lengths, L: int) -> dict:
    """The token ledger of [vllbc] Table 4-1 for samples ``lengths`` at capacity L."""
    N, T = len(lengths), sum(lengths)
    fixed = N * L
    packs = packs_lower_bound(lengths, L)
    packed = packs * L
    return {
        "T": T, "fixed": fixed, "padding": fixed - T, "waste": (fixed - T) / fixed,
        "packs": packs, "packed": packed, "pack_padding": packed - T,
        "pack_waste": (packed - T) / packed, "saved": fixed - packed,
        "saved_frac": (fixed - packed) / fixed,
        "score_elements_fixed": N * L * L // 2,
        "score_elements_packed": sum(l * l for l in lengths) // 2,
    }


def dense_slots(lengths) -> int:
    """Padded to the longest sample: B * L_max^2 score slots."""
    return len(lengths) * max(lengths) ** 2


def segment_slots(lengths) -> int:
    return sum(l * l for l in lengths)


def whole_pack_slots(lengths) -> int:
    return sum(lengths) ** 2


def causal_pairs(lengths) -> int:
    """Allowed (i, j) pairs with j <= i inside each segment: sum l (l + 1) / 2."""
    return sum(l * (l + 1) // 2 for l in lengths)


def token_slots_padded(lengths) -> int:
    return len(lengths) * max(lengths)


def useful_flops(lengths, heads: int, head_dim: int, causal: bool = True) -> int:
    """4 d H per allowed pair: 2 d for q.k plus 2 d for the p * v accumulate."""
    pairs = causal_pairs(lengths) if causal else segment_slots(lengths)
    return 4 * head_dim * heads * pairs
