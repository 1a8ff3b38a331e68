"""Oracle for the packed cross-entropy: loss sum, target count, per-segment sums.

Test infrastructure only (see the package docstring).  Plain fp64 numpy,
following the pages:

  [charlestar] "cross-boundary prediction pairs": from the [T, vocab] logits,
      cross-entropy summed over the valid targets (reduction "sum", ignore
      index -100) and the count of valid targets, kept as a sum and a count
      rather than a mean; no class weights, no label smoothing.  With the
      pre-shifted labels of pack_build (label[i] is the token that row i's
      logits predict, the ignore index on each segment's last row and on pad
      segments) row i's logits pair with label[i] directly; the page's own
      form sets each segment start's label to the ignore index and shifts by
      one, which pairs the same rows with the same targets.
  [charlestar] "packing should not choose the weight of long samples": the
      token average sum_r S_r / sum_r n_r and the sample average
      (1/B) sum_r S_r / n_r from per-sample loss sums S_r and target counts n_r.

Per target: loss_i = log(sum_v exp(z_iv)) - z_i,y_i, the log-sum-exp taken
after subtracting the row maximum (the usual stable form of the same value).
The gradient of the loss sum with respect to row i's logits is
softmax(z_i) - onehot(y_i) for a valid target and zero for an ignored one; the
optional ``scale`` multiplies it (a caller's 1/N or W/N from the pages'
"distributed denominator" section).

A label outside [0, vocab) that is not the ignore index is not a target: the
row adds nothing and ERR_LABEL is reported (PyTorch raises instead).
"""

from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100
ERR_LABEL = 256          # a label outside [0, vocab) that is not the ignore index


def _as_f64(logits) -> np.ndarray:
    """bf16 bit patterns (uint16) or floating values -> float64 [T, V]."""
    a = np.asarray(logits)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def row_losses(logits, labels, ignore_index: int = IGNORE_INDEX, chunk: int = 1024):
    """Per-row loss (0 where the row is not a target), target mask and error bits."""
    labels = np.asarray(labels, np.int64)
    T = labels.shape[0]
    V = np.asarray(logits).shape[1]
    valid = (labels != ignore_index) & (labels >= 0) & (labels < V)
    err = ERR_LABEL if ((labels != ignore_index) & ~valid).any() else 0
    loss = np.zeros(T, np.float64)
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        z = _as_f64(np.asarray(logits)[a:b])
        m = z.max(axis=1)
        lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        sel = valid[a:b]
        rows = np.nonzero(sel)[0]
        loss[a + rows] = lse[rows] - z[rows, labels[a + rows]]
    return loss, valid, err


def packed_loss(logits, labels, cu=None, ignore_index: int = IGNORE_INDEX) -> dict:
    """loss_sum (fp64), target_count (int), row_loss [T], and with ``cu`` the
    per-segment loss sums and target counts over [cu_r, cu_{r+1})."""
    loss, valid, err = row_losses(logits, labels, ignore_index)
    out = {"row_loss": loss, "valid": valid, "loss_sum": float(loss.sum()),
           "target_count": int(valid.sum()), "err": err}
    if cu is not None:
        cu = np.asarray(cu, np.int64)
        n = cu.shape[0] - 1
        seg_loss = np.zeros(n, np.float64)
        seg_count = np.zeros(n, np.int64)
        for r in range(n):
            s, e = int(cu[r]), int(cu[r + 1])
            seg_loss[r] = loss[s:e].sum()
            seg_count[r] = int(valid[s:e].sum())
        out["seg_loss"], out["seg_count"] = seg_loss, seg_count
    return out


def loss_grad(logits, labels, scale: float = 1.0, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """scale * d(loss_sum)/d(logits), fp64 [T, V]."""
    labels = np.asarray(labels, np.int64)
    z = _as_f64(logits)
    T, V = z.shape
    valid = (labels != ignore_index) & (labels >= 0) & (labels < V)
    g = np.zeros((T, V), np.float64)
    rows = np.nonzero(valid)[0]
    if rows.size:
        zr = z[rows]
        m = zr.max(axis=1, keepdims=True)
        e = np.exp(zr - m)
        p = e / e.sum(axis=1, keepdims=True)
        p[np.arange(rows.size), labels[rows]] -= 1.0
        g[rows] = p
    return scale * g


def token_average(seg_loss, seg_count) -> float:
    """sum_r S_r / sum_r n_r ([charlestar] loss weighting)."""
    return float(np.sum(seg_loss) / np.sum(seg_count))


def sample_average(seg_loss, seg_count) -> float:
    """(1/B) sum_r S_r / n_r over samples with n_r > 0."""
    seg_loss, seg_count = np.asarray(seg_loss, np.float64), np.asarray(seg_count)
    keep = seg_count > 0
    return float(np.mean(seg_loss[keep] / seg_count[keep]))
