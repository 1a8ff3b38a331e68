"""Oracle for block-diagonal (causal) attention over a packed THD buffer, fp64.

Test infrastructure only (see the package docstring).

Definition followed ([charlestar] "EOS is content": allow() and the masked
softmax equation; [compass] "cross-contamination": the block-diagonal mask):
  allow(i, j) = seg(i) == seg(j) and j <= i   (causal)
  allow(i, j) = seg(i) == seg(j)              (non-causal: a reading; the pages
                                               define only the causal mask)
  O = softmax(Q K^T / sqrt(d) + M) V,  M = 0 where allowed, -inf elsewhere.

Three forms are provided:
  attention_rows   the C loop (attn_oracle.c) for any list of query rows, used
                   at full size on sampled rows and for the CPU baseline;
  attention_brute  an explicit T x T additive mask in numpy, for tiny T
                   ([charlestar] "varlen interface": an explicit 9x9 block-causal
                   mask defines the correct result);
  attention_unpacked  each segment run alone as one ordinary sequence
                   ([m020] "08": packed vs per-sample execution;
                   [charlestar] "change A, not B").
the padded-storage form (Megatron's cu_seqlens_padded, which [vllbc] "five
steps" names beside cu_seqlens: logical boundaries apart from storage
offsets):
  attention_padded / attention_bwd_padded  segment r's L_r tokens sit at
                   storage rows [cu_padded[r], cu_padded[r] + L_r); the rest of
                   its slot up to cu_padded[r+1] is padding that no row sees.
                   Reading (the pages leave it open): real tokens at the start
                   of their slot; a padding row has no keys, its output and
                   gradients are 0 and its LSE is -inf;
  allow_matrix_padded + attention_brute_masked  the same as an explicit
                   storage x storage mask, for tiny T;
the inference-prefill form ([m020] "07 train vs infer": independent requests
through a varlen kernel, each with its own KV):
  attention_qk     separate query and key boundaries cu_q / cu_k (request r
                   has Lq_r queries over Lk_r keys, e.g. a cached prefix plus
                   the new tokens) and grouped key/value heads (query head h
                   reads kv head h // (H / Hkv)).  Causal alignment (a
                   reading: [charlestar] "varlen interface" warns that the
                   equal-length lower triangle does not carry over to
                   non-square Q/K and leaves the convention to the library
                   version): bottom-right, query a of a request sees keys
                   b <= a + Lk - Lq, so its last query sees every key and
                   Lq = Lk is the ordinary causal mask.  A query that sees no
                   key outputs 0 with LSE -inf;
and the gradients of that definition:
  attention_bwd    dQ, dK, dV for an upstream dO, per segment and head (the C
                   loop oracle_attn_bwd_segment; the softmax-Jacobian formulas
                   are written out in attn_oracle.c).  The pages print no
                   backward formulas; this is the calculus of their forward
                   definition, pinned by autograd and finite differences.
"""

from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .pack import segment_of
from .rope import bf16_bits_to_f64

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIBPATH)
        p = ctypes.c_void_p
        lib.oracle_attn_rows.argtypes = [p, p, p, p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, p, ctypes.c_int64,
                                         p, p, p]
        lib.oracle_attn_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def attention_rows(q, k, v, cu, rows, causal: bool = True, threads: int = 1):
    """fp64 outputs [n, H, d] and lse [n, H] for query ``rows`` (all heads).

    q, k, v: uint16 bf16 bits [T, H, d].  Rows are split over ``threads`` host
    threads; each thread runs the same plain loop on its own rows.
    """
    lib = _load()
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    cu32 = np.ascontiguousarray(cu, np.int32)
    rows = np.ascontiguousarray(rows, np.int64)
    T, H, d = q.shape
    nseg = cu32.shape[0] - 1
    maxlen = int((cu32[1:].astype(np.int64) - cu32[:-1]).max()) if nseg else 1
    out = np.empty((rows.shape[0], H, d), np.float64)
    lse = np.empty((rows.shape[0], H), np.float64)

    def run(lo, hi):
        if hi <= lo:
            return 0
        scratch = np.empty(max(maxlen, 1), np.float64)
        sub_rows = rows[lo:hi]
        o = out[lo:hi]
        ls = lse[lo:hi]
        return lib.oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(cu32), nseg, H, d,
                                    int(bool(causal)), _ptr(sub_rows), hi - lo,
                                    _ptr(o), _ptr(ls), _ptr(scratch))

    n = rows.shape[0]
    threads = max(1, min(int(threads), n))
    if threads == 1:
        rc = [run(0, n)]
    else:
        # interleave work in small chunks so long and short rows spread evenly
        chunk = max(1, min(64, n // (threads * 8) or 1))
        bounds = [(s, min(n, s + chunk)) for s in range(0, n, chunk)]
        with ThreadPoolExecutor(threads) as ex:
            rc = list(ex.map(lambda b: run(*b), bounds))
    if any(rc):
        raise ValueError("a query row lies outside every segment")
    return out, lse


def attention(q, k, v, cu, causal: bool = True, threads: int = 1):
    """Every row of the buffer."""
    T = q.shape[0]
    return attention_rows(q, k, v, cu, np.arange(T, dtype=np.int64), causal, threads)


def _as_f64(x):
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else np.ascontiguousarray(x, np.float64)


def allow_matrix(cu, causal: bool = True) -> np.ndarray:
    """bool [T, T]: allow(i, j) from segment ids and positions, element by element."""
    cu = np.asarray(cu, np.int64)
    T = int(cu[-1])
    seg = [segment_of(cu, i) for i in range(T)]
    A = np.zeros((T, T), bool)
    for i in range(T):
        for j in range(T):
            A[i, j] = seg[i] == seg[j] and (j <= i or not causal)
    return A


def attention_brute(q, k, v, cu, causal: bool = True):
    """Explicit additive mask: softmax(Q K^T / sqrt(d) + M) V per head, fp64 (tiny T).

    Inputs are bf16 bit patterns (uint16) or floating arrays [T, H, d]."""
    Q, K, V = (_as_f64(x) for x in (q, k, v))
    T, H, d = Q.shape
    M = np.where(allow_matrix(cu, causal), 0.0, -np.inf)
    out = np.empty((T, H, d))
    lse = np.empty((T, H))
    for h in range(H):
        S = Q[:, h, :] @ K[:, h, :].T / np.sqrt(d) + M
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        out[:, h, :] = (E @ V[:, h, :]) / E.sum(axis=1, keepdims=True)
        lse[:, h] = m[:, 0] + np.log(E.sum(axis=1))
    return out, lse


def attention_unpacked(q, k, v, cu, causal: bool = True, threads: int = 1):
    """Each segment alone, as a standalone sequence with cu = [0, L]."""
    cu = np.asarray(cu, np.int64)
    outs, lses = [], []
    for r in range(cu.shape[0] - 1):
        s, e = int(cu[r]), int(cu[r + 1])
        o, ls = attention(q[s:e], k[s:e], v[s:e], np.asarray([0, e - s]), causal, threads)
        outs.append(o)
        lses.append(ls)
    return np.concatenate(outs), np.concatenate(lses)


def attention_bwd(q, k, v, dout, cu, causal: bool = True, threads: int = 1, heads=None, segments=None):
    """fp64 gradients (dq, dk, dv), each [T, H, d], of the attention above for
    upstream gradient ``dout`` (the C loop ``oracle_attn_bwd_segment`` per
    segment and head; the formulas are in attn_oracle.c).

    Inputs are bf16 bit patterns (uint16) or floating arrays [T, H, d].
    ``heads`` / ``segments`` restrict the work to those heads / segment
    indices (other entries of the outputs stay NaN).
    """
    lib = _load()
    if not hasattr(lib, "_bwd_ready"):
        p = ctypes.c_void_p
        lib.oracle_attn_bwd_segment.argtypes = [p, p, p, p, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int64, ctypes.c_int32, p, p, p, p]
        lib.oracle_attn_bwd_segment.restype = None
        lib._bwd_ready = True
    Q, K, V, G = (_as_f64(x) for x in (q, k, v, dout))
    T, H, d = Q.shape
    cu = np.asarray(cu, np.int64)
    heads = range(H) if heads is None else list(heads)
    segments = range(cu.shape[0] - 1) if segments is None else list(segments)
    dq, dk, dv = (np.full((T, H, d), np.nan) for _ in range(3))
    ld = H * d
    jobs = [(r, h) for r in segments for h in heads]

    def run(job):
        r, h = job
        s, e = int(cu[r]), int(cu[r + 1])
        n = e - s
        if n <= 0:
            return
        scratch = np.empty(2 * n + d, np.float64)
        off = (s * H + h) * d * 8            # byte offset of (row s, head h)
        base = lambda a: ctypes.c_void_p(a.ctypes.data + off)  # noqa: E731
        lib.oracle_attn_bwd_segment(base(Q), base(K), base(V), base(G), n, d, ld, int(bool(causal)),
                                    base(dq), base(dk), base(dv), _ptr(scratch))

    threads = max(1, min(int(threads), len(jobs)))
    if threads == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return dq, dk, dv


def storage_rows(cu, cu_padded) -> np.ndarray:
    """Storage row of every real token, in order: token t of segment r (the
    (t - cu[r])-th of its segment) sits at cu_padded[r] + t - cu[r]."""
    cu = np.asarray(cu, np.int64)
    cp = np.asarray(cu_padded, np.int64)
    out = []
    for r in range(cu.shape[0] - 1):
        out.extend(range(int(cp[r]), int(cp[r] + cu[r + 1] - cu[r])))
    return np.asarray(out, np.int64)


def attention_padded(q, k, v, cu, cu_padded, causal: bool = True, threads: int = 1):
    """fp64 out [Ts, H, d] and lse [Ts, H] over storage rows (Ts = q.shape[0]);
    real rows as ``attention`` on the compact buffer, padding rows 0 / -inf."""
    idx = storage_rows(cu, cu_padded)
    Ts, H, d = np.asarray(q).shape
    o, ls = attention(np.asarray(q)[idx], np.asarray(k)[idx], np.asarray(v)[idx], cu, causal, threads)
    out = np.zeros((Ts, H, d))
    lse = np.full((Ts, H), -np.inf)
    out[idx], lse[idx] = o, ls
    return out, lse


def attention_bwd_padded(q, k, v, dout, cu, cu_padded, causal: bool = True, threads: int = 1, heads=None,
                         segments=None):
    """Gradients over storage rows: real rows as ``attention_bwd`` on the
    compact buffer, padding rows 0 (NaN outside ``heads`` / ``segments``)."""
    idx = storage_rows(cu, cu_padded)
    Ts = np.asarray(q).shape[0]
    g = attention_bwd(np.asarray(q)[idx], np.asarray(k)[idx], np.asarray(v)[idx], np.asarray(dout)[idx], cu,
                      causal, threads, heads, segments)
    outs = []
    for a in g:
        full = np.zeros((Ts,) + a.shape[1:])
        if heads is not None:
            keep = np.zeros(a.shape[1], bool)
            keep[list(heads)] = True
            full[:, ~keep] = np.nan
        full[idx] = a
        outs.append(full)
    return tuple(outs)


def allow_matrix_padded(cu, cu_padded, total_rows: int, causal: bool = True) -> np.ndarray:
    """bool [Ts, Ts] over storage rows: i and j real rows of the same slot, and
    j <= i when causal; padding rows allow nothing."""
    cu = np.asarray(cu, np.int64)
    cp = np.asarray(cu_padded, np.int64)
    slot = np.full(total_rows, -1)
    for r in range(cu.shape[0] - 1):
        slot[cp[r]:cp[r] + cu[r + 1] - cu[r]] = r
    A = np.zeros((total_rows, total_rows), bool)
    for i in range(total_rows):
        for j in range(total_rows):
            A[i, j] = slot[i] >= 0 and slot[i] == slot[j] and (j <= i or not causal)
    return A


def attention_brute_masked(q, k, v, allow):
    """softmax(Q K^T / sqrt(d) + M) V for an explicit bool mask; a row that
    allows nothing gets output 0 and LSE -inf.  fp64, tiny T."""
    Q, K, V = (_as_f64(x) for x in (q, k, v))
    T, H, d = Q.shape
    allow = np.asarray(allow, bool)
    M = np.where(allow, 0.0, -np.inf)
    has = allow.any(axis=1)
    out = np.zeros((T, H, d))
    lse = np.full((T, H), -np.inf)
    for h in range(H):
        S = Q[has, h, :] @ K[:, h, :].T / np.sqrt(d) + M[has]
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        out[has, h, :] = (E @ V[:, h, :]) / E.sum(axis=1, keepdims=True)
        lse[has, h] = m[:, 0] + np.log(E.sum(axis=1))
    return out, lse


def attention_qk(q, k, v, cu_q, cu_k, causal: bool = True, rows=None):
    """fp64 out [Tq, H, d], lse [Tq, H] for q [Tq, H, d] over k, v [Tk, Hkv, d]
    (H a multiple of Hkv), request r = queries [cu_q[r], cu_q[r+1]) over keys
    [cu_k[r], cu_k[r+1]); plain per request and head.  ``rows``: compute only
    those query rows (the others stay 0 / -inf)."""
    Q, K, V = (_as_f64(x) for x in (q, k, v))
    Tq, H, d = Q.shape
    Hkv = K.shape[1]
    group = H // Hkv
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    out = np.zeros((Tq, H, d))
    lse = np.full((Tq, H), -np.inf)
    rowset = None if rows is None else {int(x) for x in rows}
    for r in range(cu_q.shape[0] - 1):
        qs, qe, ks, ke = int(cu_q[r]), int(cu_q[r + 1]), int(cu_k[r]), int(cu_k[r + 1])
        Lq, Lk = qe - qs, ke - ks
        for a in range(Lq):
            if rowset is not None and (qs + a) not in rowset:
                continue
            nvis = min(Lk, a + Lk - Lq + 1) if causal else Lk      # keys 0 .. nvis-1
            if nvis <= 0:
                continue
            for h in range(H):
                hk = h // group
                sc = K[ks:ks + nvis, hk, :] @ Q[qs + a, h, :] / np.sqrt(d)
                m = sc.max()
                e = np.exp(sc - m)
                out[qs + a, h, :] = e @ V[ks:ks + nvis, hk, :] / e.sum()
                lse[qs + a, h] = m + np.log(e.sum())
    return out, lse
