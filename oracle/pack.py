"""Oracle for the packing metadata: prefix sums, segment ids, positions, labels.

Test infrastructure only (see the package docstring).  Every function follows
the pages step by step:

  [charlestar] "nine tokens, three identities": cu_seqlens is the prefix sum of
      the sample lengths, segment r is [cu_r, cu_{r+1}), the local position of
      token i in segment r is p_i = i - cu_r, and max_seqlen is the longest
      segment (4 for [3,2,4], not the total 9).  The same section lists what a
      caller must guarantee: cu[0] == 0, strictly increasing, cu[-1] == total,
      max_seqlen equal to the largest difference, int32-representable values.
  [vllbc] "three things: concatenate, cut, mask": cu_seqlens = [0, l1, l1+l2, ...].
  [m020] "06 positions and labels": next-token targets aligned to the input
      position; the last token of a sample predicts nothing.
  [charlestar] "cross-boundary prediction pairs": the two label conventions
      and the valid-target count sum_r (L_r - 1).
  [compass] "implementation notes": the pack tail is its own segment whose
      labels are all -100.

Reading adopted where the pages leave a choice open: labels are pre-shifted,
``label[i] = token[i+1]`` when i+1 lies in the same non-pad segment, else the
ignore index; positions inside a pad segment are ``i - cu[seg(i)]`` like every
other segment (the page's pack builder writes zeros there; no loss reads them).
"""

from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100

# device error bits, as documented for the library's error word
ERR_CU0 = 1              # cu[0] != 0
ERR_NOT_INCREASING = 2   # some cu[r+1] <= cu[r] (a segment of length <= 0)
ERR_TOTAL = 4            # cu[nseg] != total_tokens
ERR_MAXSEQ = 8           # a segment is longer than max_seqlen
ERR_LENGTH = 16          # a sample length <= 0 given to pack_build
ERR_MISMATCH = 32        # cu disagrees with the sample lengths it should come from
ERR_RANGE = 64           # the total does not fit in int32


def cu_seqlens(lengths) -> np.ndarray:
    """cu[0] = 0, cu[r+1] = cu[r] + l_r, as int64 so overflow stays visible."""
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(lengths.shape[0] + 1, np.int64)
    for r in range(lengths.shape[0]):
        cu[r + 1] = cu[r] + lengths[r]
    return cu


def pack_build(lengths, tokens=None, is_pad=None, ignore_index: int = IGNORE_INDEX) -> dict:
    """Packing metadata for one buffer.

    Returns cu_seqlens [n+1], segment_ids [T], position_ids [T], shifted_labels [T]
    (int32), loss_mask [T] (uint8), num_targets (int) and max_seqlen (int), plus
    the error bits the device library must raise for the same lengths.
    """
    lengths = np.asarray(lengths, np.int64)
    n = int(lengths.shape[0])
    is_pad = np.zeros(n, np.uint8) if is_pad is None else np.asarray(is_pad, np.uint8)
    err = 0
    if n and int(lengths.min()) <= 0:
        err |= ERR_LENGTH
    cu = cu_seqlens(lengths)
    T = int(cu[-1])
    if T > np.iinfo(np.int32).max:
        err |= ERR_RANGE
    max_seqlen = int(lengths.max()) if n else 0
    out = {"cu_seqlens": cu.astype(np.int32) if not err & ERR_RANGE else cu,
           "max_seqlen": max_seqlen, "error": err}
    if err:
        return out
    seg = np.empty(T, np.int32)
    pos = np.empty(T, np.int32)
    label = np.full(T, ignore_index, np.int32)
    for r in range(n):
        s, e = int(cu[r]), int(cu[r + 1])
        seg[s:e] = r
        pos[s:e] = np.arange(e - s, dtype=np.int32)           # p_i = i - cu_r
        if tokens is not None and not is_pad[r]:
            label[s:e - 1] = np.asarray(tokens[s + 1:e], np.int32)  # i+1 in the same segment
    loss_mask = (label != ignore_index).astype(np.uint8)
    out.update(segment_ids=seg, position_ids=pos, shifted_labels=label,
               loss_mask=loss_mask, num_targets=int(loss_mask.astype(np.int64).sum()))
    return out


def validate_cu(cu, total_tokens: int, max_seqlen: int, lengths=None) -> int:
    """Error bits for a caller-supplied cu_seqlens (the preconditions listed above)."""
    cu = np.asarray(cu, np.int64)
    err = 0
    if cu.shape[0] < 2:
        return ERR_TOTAL
    if cu[0] != 0:
        err |= ERR_CU0
    d = cu[1:] - cu[:-1]
    if (d <= 0).any():
        err |= ERR_NOT_INCREASING
    if cu[-1] != total_tokens:
        err |= ERR_TOTAL
    if (d > max_seqlen).any():
        err |= ERR_MAXSEQ
    if lengths is not None:
        lengths = np.asarray(lengths, np.int64)
        if lengths.shape[0] != d.shape[0] or (lengths != d).any():
            err |= ERR_MISMATCH
    return err


def segment_of(cu, i: int) -> int:
    """The r with cu[r] <= i < cu[r+1] (linear scan)."""
    cu = np.asarray(cu, np.int64)
    for r in range(cu.shape[0] - 1):
        if cu[r] <= i < cu[r + 1]:
            return r
    raise IndexError(i)


def positions_from_cu(cu) -> np.ndarray:
    """p_i = i - cu[seg(i)] for every token, from a cu_seqlens array."""
    cu = np.asarray(cu, np.int64)
    T = int(cu[-1])
    pos = np.empty(T, np.int64)
    for r in range(cu.shape[0] - 1):
        s, e = int(cu[r]), int(cu[r + 1])
        pos[s:e] = np.arange(e - s)
    return pos
