"""Seeded synthetic workloads for packed variable-length causal attention.

Page tags used in citations (the pages are the specification):
  [vllbc]      blog.vllbc.top  "long-context training: remove padding"
  [compass]    brenchcc.github.io/llm-compass  "Sequence Packing" (SFT chapter)
  [m020]       xuujii.github.io/ai-infra-kb  M020 "length grouping, de-padding and packing"
  [opworld]    operatorworld.com  "packing and document boundaries"
  [charlestar] charlestar.github.io  "sequence packing and variable-length attention"

Every random draw comes from ``numpy.random.default_rng([cfg_id, stream, seed])``
(PCG64).  Streams: 0 = sample lengths, 1 = token ids, 2/3/4 = q/k/v, 5 = an upstream
gradient of the attention output, 6 = logits for the packed cross-entropy,
7 = prefill request lengths, 8/9/10 = prefill q/k/v.  q/k/v are
standard normal float32 values rounded to bf16 (round to nearest even) and are
carried as uint16 bit patterns, shape ``[T, H, d]`` (THD, no batch dim).

The module holds no step of the method itself; it emits sample lengths, pad
flags and tokens.  Prefix sums, positions and labels are computed by the oracle
and by the GPU library from these lengths.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

EOS_ID = 2          # every real sample ends in an end-of-sequence token
PAD_ID = 0          # id written into pad-tail segments
VOCAB_LO, VOCAB_HI = 3, 32000

CONFIG_NAMES = ("tiny", "sft", "pretrain", "longctx", "short")
_CFG_ID = {name: i for i, name in enumerate(CONFIG_NAMES)}


def _rng(cfg_id: int, stream: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([cfg_id, stream, seed])


@dataclasses.dataclass
class Workload:
    """One packed buffer: segment lengths in buffer order plus attention shape."""

    name: str
    cfg_id: int
    seed: int
    lengths: np.ndarray          # int32 [nseg], all > 0, in buffer order
    is_pad: np.ndarray           # uint8 [nseg], 1 for pad-tail segments
    heads: int
    head_dim: int
    causal: bool = True
    rope_base: float = 10000.0
    pad_len: int = 0             # L of the padded-SBHD comparison layout
    note: str = ""

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def nseg(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def real_lengths(self) -> np.ndarray:
        return self.lengths[self.is_pad == 0]

    def tokens(self) -> np.ndarray:
        return token_ids(self)

    def qkv(self, which: str = "qkv") -> list[np.ndarray]:
        return [qkv_bits(self, w) for w in which]

    def describe(self) -> dict:
        rl = self.real_lengths
        return {
            "workload": self.name,
            "total_tokens": self.total_tokens,
            "real_tokens": int(rl.sum()),
            "segments": self.nseg,
            "pad_segments": int(self.is_pad.sum()),
            "max_seqlen": int(self.lengths.max()),
            "heads": self.heads,
            "head_dim": self.head_dim,
            "causal": self.causal,
            "seed": self.seed,
        }


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------ length recipes

def _ffd(lengths: np.ndarray, cap: int) -> list[list[int]]:
    """First-fit decreasing into bins of ``cap`` tokens.

    Samples are visited longest first with a stable order for ties, and each
    goes into the first bin, in creation order, that still has room; samples
    stay in insertion order inside a bin ([compass] "implementation notes"
    code, first-fit packing; [opworld] "efficiency ledger" names FFD).
    """
    order = np.argsort(-lengths, kind="stable")
    bins: list[list[int]] = []
    fill: list[int] = []
    for idx in order:
        L = int(lengths[idx])
        for b in range(len(bins)):
            if fill[b] + L <= cap:
                bins[b].append(int(idx))
                fill[b] += L
                break
        else:
            bins.append([int(idx)])
            fill.append(L)
    return bins


def _sft_lengths(seed: int, packs: int = 8, cap: int = 4096, median: float = 300.0,
                 sigma: float = 1.0, lo: int = 16):
    """SFT packing: lognormal sample lengths packed by FFD into ``packs`` bins.

    The drawn prefix grows while FFD still needs at most ``packs`` bins.  Each
    bin's unused tail becomes its own pad segment, the tail layout of
    [compass] "implementation notes" (pack builder pads and closes the prefix).
    """
    rng = _rng(_CFG_ID["sft"], 0, seed)
    z = rng.standard_normal(100000)
    draws = np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, cap).astype(np.int64)
    n = 1
    best = _ffd(draws[:1], cap)
    while n < draws.shape[0]:
        trial = _ffd(draws[: n + 1], cap)
        if len(trial) > packs:
            break
        best = trial
        n += 1
    lengths, is_pad = [], []
    for b in best:
        used = 0
        for idx in b:
            lengths.append(int(draws[idx]))
            is_pad.append(0)
            used += int(draws[idx])
        if used < cap:
            lengths.append(cap - used)
            is_pad.append(1)
    for _ in range(packs - len(best)):
        lengths.append(cap)
        is_pad.append(1)
    return np.asarray(lengths, np.int32), np.asarray(is_pad, np.uint8)


def _pretrain_lengths(windows: int = 16, docs: int = 10, doc_len: int = 400, rem: int = 96):
    """Fixed pretraining windows: ``docs`` documents of ``doc_len`` plus a remainder.

    16 x (10 x 400 + 96) = 65,536 tokens; the 4k-window, ten-400-token-document
    example of [opworld] "pitfall one: cross-document attention".
    """
    one = [doc_len] * docs + ([rem] if rem else [])
    lengths = np.asarray(one * windows, np.int32)
    return lengths, np.zeros(lengths.shape, np.uint8)


def _longctx_lengths(seed: int, total: int = 131072, p_long: float = 0.1,
                     long_lo: int = 8192, long_hi: int = 32768, median: float = 512.0,
                     sigma: float = 1.2, lo: int = 8):
    """Long-context pack filled greedily to exactly ``total`` tokens.

    Each draw is uniform in [long_lo, long_hi] with probability ``p_long``,
    otherwise lognormal(median, sigma) with a floor of ``lo``; the last draw is
    clipped so the buffer holds exactly ``total`` tokens ([vllbc] intro: the
    131,072-slot long-context waste example).
    """
    rng = _rng(_CFG_ID["longctx"], 0, seed)
    remaining, out = total, []
    while remaining > 0:
        if rng.random() < p_long:
            L = int(rng.integers(long_lo, long_hi, endpoint=True))
        else:
            L = max(lo, int(np.rint(np.exp(math.log(median) + sigma * rng.standard_normal()))))
        L = min(L, remaining)
        out.append(L)
        remaining -= L
    lengths = np.asarray(out, np.int32)
    return lengths, np.zeros(lengths.shape, np.uint8)


def _short_lengths(seed: int, total: int = 65536, lo: int = 8, hi: int = 128):
    """Short-segment stress: uniform [lo, hi] lengths until exactly ``total`` tokens.

    The last segment is clipped and may be shorter than ``lo``; the 128-token
    BERT-like maximum of [vllbc] "padding waste" (GLUE-CoLA at length 128).
    """
    rng = _rng(_CFG_ID["short"], 0, seed)
    remaining, out = total, []
    while remaining > 0:
        L = min(int(rng.integers(lo, hi, endpoint=True)), remaining)
        out.append(L)
        remaining -= L
    lengths = np.asarray(out, np.int32)
    return lengths, np.zeros(lengths.shape, np.uint8)


def make_workload(name: str, seed: int = 0, *, heads: int | None = None,
                  scale: str = "full", **kw) -> Workload:
    """Build one named workload.

    ``scale="full"`` gives the sizes the bench runs.  ``scale="small"`` keeps
    each length recipe but shrinks the buffer and the head count so the fp64
    oracle finishes every element in seconds while the input still spans
    several tiles and ragged tails.  Keyword arguments override the recipe.
    """
    if name not in _CFG_ID:
        raise KeyError(f"unknown workload {name!r}; choose from {CONFIG_NAMES}")
    cid = _CFG_ID[name]
    small = scale == "small"
    if name == "tiny":
        lengths = np.asarray(kw.get("lengths", [3, 2, 4]), np.int32)
        is_pad = np.zeros(lengths.shape, np.uint8)
        H, d, pad_len = 2, 64, int(lengths.max())
        note = "lengths [3,2,4]: the nine-token example of [charlestar]"
    elif name == "sft":
        args = dict(packs=2, cap=1024, median=150.0) if small else {}
        args.update(kw)
        lengths, is_pad = _sft_lengths(seed, **args)
        H, d, pad_len = (2 if small else 32), 128, args.get("cap", 4096)
        note = "lognormal sample lengths packed first-fit-decreasing, pad tails as segments"
    elif name == "pretrain":
        args = dict(windows=2) if small else {}
        args.update(kw)
        lengths, is_pad = _pretrain_lengths(**args)
        H, d, pad_len = (2 if small else 32), 128, 4096
        note = "windows of 10 x 400-token documents plus a 96-token remainder"
    elif name == "longctx":
        args = dict(total=8192, long_lo=1024, long_hi=4096, median=256.0) if small else {}
        args.update(kw)
        lengths, is_pad = _longctx_lengths(seed, **args)
        H, d, pad_len = (2 if small else 32), 128, args.get("total", 131072)
        note = "one long-context buffer: 10% long segments, lognormal rest"
    else:
        args = dict(total=4096) if small else {}
        args.update(kw)
        lengths, is_pad = _short_lengths(seed, **args)
        H, d, pad_len = (2 if small else 16), 64, args.get("hi", 128)
        note = "thousands of short uniform segments"
    if heads is not None:
        H = heads
    return Workload(name=name, cfg_id=cid, seed=seed, lengths=lengths, is_pad=is_pad,
                    heads=H, head_dim=d, pad_len=pad_len, note=note)


# ------------------------------------------------------------- token / qkv

def token_ids(w: Workload) -> np.ndarray:
    """int32 [T]: uniform ids in [3, 32000); each real sample ends in EOS, pads are 0."""
    rng = _rng(w.cfg_id, 1, w.seed)
    t = rng.integers(VOCAB_LO, VOCAB_HI, size=w.total_tokens, dtype=np.int64).astype(np.int32)
    start = 0
    for L, pad in zip(w.lengths.tolist(), w.is_pad.tolist()):
        if pad:
            t[start:start + L] = PAD_ID
        else:
            t[start + L - 1] = EOS_ID
        start += L
    return t


def qkv_bits(w: Workload, which: str, chunk: int = 1 << 24) -> np.ndarray:
    """uint16 [T, H, d] bf16 bit patterns of N(0,1) draws for ``which`` in
    'q', 'k', 'v' or 'g' (an upstream gradient for the attention output)."""
    stream = {"q": 2, "k": 3, "v": 4, "g": 5}[which]
    rng = _rng(w.cfg_id, stream, w.seed)
    n = w.total_tokens * w.heads * w.head_dim
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(w.total_tokens, w.heads, w.head_dim)


def logits_bits(w: Workload, vocab: int, sigma: float = 2.0, rows: int | None = None,
                chunk: int = 1 << 24) -> np.ndarray:
    """uint16 [rows or T, vocab] bf16 bit patterns of N(0, sigma^2) logits."""
    rng = _rng(w.cfg_id, 6, w.seed)
    T = w.total_tokens if rows is None else rows
    n = T * vocab
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32) * np.float32(sigma))
    return out.reshape(T, vocab)


@dataclasses.dataclass
class Prefill:
    """An inference prefill of independent requests: request r brings
    new_len[r] new tokens (its queries) after a cached prefix of
    prefix_len[r] tokens; its keys are the prefix plus the new tokens."""

    name: str
    seed: int
    new_len: np.ndarray          # int32 [n] = Lq
    prefix_len: np.ndarray       # int32 [n]
    heads: int
    kv_heads: int
    head_dim: int

    @property
    def lq(self) -> np.ndarray:
        return self.new_len.astype(np.int64)

    @property
    def lk(self) -> np.ndarray:
        return (self.new_len.astype(np.int64) + self.prefix_len)

    @property
    def total_q(self) -> int:
        return int(self.lq.sum())

    @property
    def total_k(self) -> int:
        return int(self.lk.sum())


def make_prefill(seed: int = 0, *, scale: str = "full") -> Prefill:
    """Requests until total_q new tokens: new lengths lognormal(median 256,
    sigma 1) clipped to [1, 2048]; cached prefixes 0 with probability 0.3,
    else uniform in [1, 4096]; 32 query heads over 8 key / value heads (the
    "full" size, 32,768 query rows) or 4 over 2 ("small", 2,048 rows)."""
    small = scale == "small"
    total = 2048 if small else 32768
    rng = np.random.default_rng([len(CONFIG_NAMES), 7, seed])
    new, pre = [], []
    while sum(new) < total:
        L = int(np.clip(np.rint(np.exp(math.log(256.0) + rng.standard_normal())), 1, 2048))
        L = min(L, total - sum(new))
        new.append(L)
        pre.append(0 if rng.random() < 0.3 else int(rng.integers(1, (1024 if small else 4096) + 1)))
    H, Hkv = (4, 2) if small else (32, 8)
    return Prefill("prefill", seed, np.asarray(new, np.int32), np.asarray(pre, np.int32), H, Hkv, 128)


def prefill_bits(pw: Prefill, which: str) -> np.ndarray:
    """uint16 bf16 bits of N(0,1): q [Tq, H, d], k / v [Tk, Hkv, d]."""
    stream = {"q": 8, "k": 9, "v": 10}[which]
    rng = np.random.default_rng([len(CONFIG_NAMES), stream, pw.seed])
    rows, heads = (pw.total_q, pw.heads) if which == "q" else (pw.total_k, pw.kv_heads)
    x = rng.standard_normal(rows * heads * pw.head_dim, dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(rows, heads, pw.head_dim)
