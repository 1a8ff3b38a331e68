"""Benchmark of the packed varlen causal attention path on one MI355X.

One step = the whole hot path over one packed batch already resident in HBM:
  pack_build (cu_seqlens, segment ids, positions, shifted labels, loss mask,
  target count) -> rope_thd_apply on q and k -> attn_plan -> varlen_attn_fwd.
Default workload (the headline line): the long-context buffer, 131,072 tokens
(10% of the samples uniform in [8192, 32768], the rest lognormal with median
512), 32 heads, head_dim 128, causal.  It is the largest configuration that
fits one GPU and the one the >= 40%-of-peak target names; the forward there
is bound by the MFMA rate.

Printed: ONE JSON line.  value = useful attention TFLOP/s over the whole step
(useful FLOPs = 4 d H per same-segment causal pair of the real samples; pad
segments are computed but not counted).  Per-kernel durations come from HIP
events recorded on the stream the kernels run on.  `roofline` is the forward
kernel's, against its binding roof.  Beside it, in the same process: the
backward (varlen_attn_bwd, not part of the step: useful FLOPs 2.5x the
forward's), the packed cross-entropy over the step's labels with [T, 32000]
logits (packed_ce_loss, not part of the step), the other workloads (SFT
packs, 4k pretraining windows, short segments) with their own rooflines, an
inference prefill through the separate-boundary forward (varlen_attn_fwd_qk),
the same kernel on the padded SBHD layout, and the fp64 CPU oracle timed on a
bounded sample of rows (all host threads), with single-thread oracle times of
the tiny, pretraining-window and short-segment workloads and of the
long-context buffer (the last two extrapolated from timed subsets, labelled).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "varlen causal attn fwd useful TFLOP/s (% bf16 MFMA peak) + effective tokens/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
# useful backward FLOPs per useful forward FLOP: five products of the forward's
# size (S = QK^T again, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q)
# against the forward's two
BWD_FLOP_RATIO = 2.5


def useful_flops(lengths, is_pad, heads, head_dim, causal=True) -> float:
    L = np.asarray(lengths, np.float64)[np.asarray(is_pad) == 0]
    pairs = (L * (L + 1) / 2).sum() if causal else (L * L).sum()
    return 4.0 * head_dim * heads * pairs


def attn_bytes(T, heads, head_dim) -> float:
    """Compulsory HBM bytes of one attention launch: read q, k, v, write o (bf16)."""
    return 4.0 * T * heads * head_dim * 2


def rope_bytes(T, heads, head_dim) -> float:
    return 2.0 * 2 * T * heads * head_dim * 2          # q and k, read + write


def pack_bytes(T, nseg) -> float:
    return T * (4 + 4 + 4 + 4 + 1) + nseg * (4 + 1 + 4)   # tokens in; seg, pos, label, mask out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counter_traffic(workload: str, root: str = ROOT):
    """HBM bytes per attention launch from the committed FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on this workload from the current kernel source
    (None otherwise: a figure taken from other code is not reported)."""
    import hashlib
    path = os.path.join(root, "profiles", f"attn_fwd_{workload}_hbm_counters.md")
    src = os.path.join(root, "packed_varlen_causal_amd", "csrc", "attn.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", " ")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if fields.get("attn_source_sha256_prefix") != sha:
        return None
    try:
        return float(fields["attention_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Inputs:
    def __init__(self, name, torch, pvc, scale="full", keep_host=False):
        from workloads import make_workload
        self.w = w = make_workload(name, scale=scale)
        dev = torch.device("cuda")
        t0 = time.time()
        q, k, v = w.qkv()
        to = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
        self.q, self.k, self.v = to(q), to(k), to(v)
        self.host_qkv = (q, k, v) if keep_host else None
        del q, k, v
        self.lengths = torch.from_numpy(w.lengths).to(dev)
        self.is_pad = torch.from_numpy(w.is_pad).to(dev)
        self.tokens = torch.from_numpy(w.tokens()).to(dev)
        self.q_rot = torch.empty_like(self.q)
        self.k_rot = torch.empty_like(self.k)
        self.T, self.H, self.D = w.total_tokens, w.heads, w.head_dim
        self.max_seqlen = int(w.lengths.max())
        self.flops = useful_flops(w.lengths, w.is_pad, w.heads, w.head_dim, w.causal)
        self.real_tokens = int(w.real_lengths.sum())
        self.out = torch.empty_like(self.q)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws = torch.empty(pvc.attn_workspace_size(self.T, w.nseg), dtype=torch.uint8, device=dev)
        log(f"[bench] {name}: T={self.T} nseg={w.nseg} H={self.H} d={self.D} inputs in {time.time() - t0:.1f}s")


def run_step(torch, pvc, x, ev=None):
    """One pass of the hot path; ev = list of 5 events to bracket the four stages."""
    rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)  # noqa: E731
    rec(0)
    meta = pvc.pack_build(x.lengths, x.tokens, x.is_pad, dev_error=x.err)
    rec(1)
    pvc.rope_thd_apply(x.q, x.k, meta["cu_seqlens"], x.w.rope_base, q_out=x.q_rot, k_out=x.k_rot,
                       dev_error=x.err)
    rec(2)
    plan = pvc.AttnPlan(meta["cu_seqlens"], x.T, x.max_seqlen, x.w.causal, dev_error=x.err, workspace=x.ws)
    rec(3)
    pvc.varlen_attn_fwd(x.q_rot, x.k_rot, x.v, plan=plan, causal=x.w.causal, out=x.out)
    rec(4)


def time_steps(torch, pvc, x, steps, warmup):
    for _ in range(warmup):
        run_step(torch, pvc, x)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        run_step(torch, pvc, x, evs[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    stage = np.asarray([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])
    if int(x.err.item()) != 0:
        raise RuntimeError(f"device error bits {pvc.error_names(int(x.err.item()))}")
    return total_ms / steps, stage.mean(axis=0)


def time_attn_only(torch, pvc, x, steps, warmup):
    meta = pvc.pack_build(x.lengths, x.tokens, x.is_pad, dev_error=x.err)
    pvc.rope_thd_apply(x.q, x.k, meta["cu_seqlens"], x.w.rope_base, q_out=x.q_rot, k_out=x.k_rot)
    plan = pvc.AttnPlan(meta["cu_seqlens"], x.T, x.max_seqlen, x.w.causal, dev_error=x.err, workspace=x.ws)
    for _ in range(warmup):
        pvc.varlen_attn_fwd(x.q_rot, x.k_rot, x.v, plan=plan, out=x.out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        pvc.varlen_attn_fwd(x.q_rot, x.k_rot, x.v, plan=plan, out=x.out)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_backward(torch, pvc, x, steps, warmup):
    """varlen_attn_bwd (dQ + dK/dV launches) on the step's rotated q, k,
    the forward's output and log-sum-exp, and a seeded N(0, 1) upstream
    gradient; bf16 gradients.  Returns ms per backward call."""
    meta = pvc.pack_build(x.lengths, x.tokens, x.is_pad, dev_error=x.err)
    pvc.rope_thd_apply(x.q, x.k, meta["cu_seqlens"], x.w.rope_base, q_out=x.q_rot, k_out=x.k_rot)
    plan = pvc.AttnPlan(meta["cu_seqlens"], x.T, x.max_seqlen, x.w.causal, dev_error=x.err, workspace=x.ws)
    out, lse = pvc.varlen_attn_fwd(x.q_rot, x.k_rot, x.v, plan=plan, return_lse=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    dout = torch.randn(x.q.shape, generator=gen, device="cuda", dtype=torch.bfloat16)
    grads = tuple(torch.empty_like(x.q) for _ in range(3))
    scratch = torch.empty(pvc.attn_bwd_scratch_size(x.T, x.H), dtype=torch.uint8, device="cuda")
    call = lambda: pvc.varlen_attn_bwd(x.q_rot, x.k_rot, x.v, out, dout, lse, plan,  # noqa: E731
                                       grads=grads, scratch=scratch)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    if int(x.err.item()) != 0:
        raise RuntimeError(f"device error bits {pvc.error_names(int(x.err.item()))}")
    ms = a.elapsed_time(b) / steps
    del out, lse, dout, grads, scratch
    bflops = BWD_FLOP_RATIO * x.flops
    return {"ms": round(ms, 4), "useful_tflops": round(bflops / (ms * 1e-3) / 1e12, 2),
            "pct_bf16_peak": round(100 * bflops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}


# Untimed backward calls before the timed ones.  Right after the forward
# steps the backward's first dozen calls run about 8% slower (1.41-1.46 ms on
# the SFT packs after 2 calls, 1.31-1.33 ms after 30).
BWD_WARMUP = 30

CE_VOCAB = 32000          # the token recipe's id range [3, 32000)


def time_ce(torch, pvc, x, steps, warmup, vocab=CE_VOCAB):
    """packed_ce_loss over the step's pre-shifted labels and [T, vocab] bf16
    logits drawn on the device from a seeded generator: loss sum + target
    count (+ per-segment sums), then the same with the fused gradient written
    in place.  Algorithmic bytes: the logits read once (2 T V), labels and
    row losses (8 T), plus 2 T V written with the gradient."""
    meta = pvc.pack_build(x.lengths, x.tokens, x.is_pad, dev_error=x.err)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    logits = torch.randn((x.T, vocab), generator=gen, device="cuda", dtype=torch.bfloat16) * 2
    ws = torch.empty(pvc.ce_workspace_size(x.T), dtype=torch.uint8, device="cuda")
    res = {"vocab": vocab, "logits": f"[{x.T}, {vocab}] bf16, N(0, 4), seeded on the device"}
    for name, grad in (("loss", None), ("loss_and_grad_inplace", "inplace")):
        call = lambda: pvc.packed_ce_loss(logits, meta["shifted_labels"], meta["cu_seqlens"],  # noqa: E731
                                          segments=True, grad=grad, grad_scale=1.0, workspace=ws,
                                          dev_error=x.err)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        nbytes = 2.0 * x.T * vocab * (2 if grad else 1) + 8.0 * x.T
        res[name] = {"ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "algorithmic_bytes": nbytes}
    if int(x.err.item()) != 0:
        raise RuntimeError(f"device error bits {pvc.error_names(int(x.err.item()))}")
    del logits, ws
    torch.cuda.empty_cache()
    return res


def time_prefill(torch, pvc, steps, warmup):
    """The prefill path on its own workload: independent requests with cached
    prefixes (separate query / key boundaries, bottom-right causal), 32 query
    heads over 8 key / value heads, d = 128.  Useful FLOPs: 4 d H per visible
    (query, key) pair."""
    from workloads import make_prefill
    pw = make_prefill()
    lq, lk = pw.lq, pw.lk
    pairs = 0
    for a_len, k_len in zip(lq.tolist(), lk.tolist()):
        # query a sees min(Lk, a + Lk - Lq + 1) keys
        a = np.arange(a_len)
        pairs += int(np.clip(a + k_len - a_len + 1, 0, k_len).sum())
    flops = 4.0 * pw.head_dim * pw.heads * pairs
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    q = torch.randn((pw.total_q, pw.heads, pw.head_dim), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((pw.total_k, pw.kv_heads, pw.head_dim), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)).cuda()
    cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)).cuda()
    plan = pvc.attn_plan_qk(cu_q, cu_k, pw.total_q, pw.total_k, int(lq.max()), int(lk.max()), True)
    out = torch.empty_like(q)
    for _ in range(warmup):
        pvc.varlen_attn_fwd_qk(q, k, v, plan=plan, out=out)
    torch.cuda.synchronize()
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for _ in range(steps):
        pvc.varlen_attn_fwd_qk(q, k, v, plan=plan, out=out)
    b_ev.record()
    torch.cuda.synchronize()
    if int(plan.dev_error.item()) != 0:
        raise RuntimeError(f"device error bits {pvc.error_names(int(plan.dev_error.item()))}")
    ms = a_ev.elapsed_time(b_ev) / steps
    nbytes = 2.0 * pw.head_dim * (2 * pw.total_q * pw.heads + 2 * pw.total_k * pw.kv_heads)
    tf = flops / (ms * 1e-3) / 1e12
    return {"requests": int(lq.size), "total_q": pw.total_q, "total_k": pw.total_k, "heads": pw.heads,
            "kv_heads": pw.kv_heads, "head_dim": pw.head_dim, "ms": round(ms, 4), "useful_tflops": round(tf, 2),
            "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "roofline_tflops": round(min(PEAK_BF16_TFLOPS, flops / nbytes * PEAK_HBM_GBPS / 1e3), 1),
            "setup": "prefixes 0 (p 0.3) or U[1, 4096], new lengths lognormal(256, 1) in [1, 2048]; "
                     "q/k/v N(0,1) seeded on the device"}


def padded_baseline(torch, pvc, x, reps=3, max_chunk_bytes=24 << 30):
    """Same kernel on padded SBHD [L, B, H, d]; large batches run in chunks of
    samples (exact: samples are independent) and the chunk times are summed."""
    w = x.w
    L = int(w.pad_len)
    real = w.real_lengths
    B = len(real)
    per_sample = 4 * L * x.H * x.D * 2
    chunk = max(1, min(B, max_chunk_bytes // per_sample))
    dev = torch.device("cuda")
    total_ms, timed = 0.0, 0
    nchunks = (B + chunk - 1) // chunk
    chunks_to_time = min(nchunks, 2 if L > 16384 else nchunks)
    for c in range(chunks_to_time):
        nb = min(chunk, B - c * chunk)
        g = torch.Generator(device=dev).manual_seed(1234 + c)
        q, k, v = (torch.randn((L, nb, x.H, x.D), device=dev, generator=g).to(torch.bfloat16)
                   for _ in range(3))
        sl = torch.from_numpy(real[c * chunk: c * chunk + nb].astype(np.int32)).to(dev)
        out = torch.empty_like(q)
        pvc.padded_attn_fwd_sbhd(q, k, v, sl, True, out=out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pvc.padded_attn_fwd_sbhd(q, k, v, sl, True, out=out)
        b.record()
        torch.cuda.synchronize()
        total_ms += a.elapsed_time(b) / reps
        timed += nb
        del q, k, v, out
        torch.cuda.empty_cache()
    ms = total_ms * B / timed
    padded_pairs = B * L * (L + 1) / 2
    real_pairs = (real.astype(np.float64) * (real + 1) / 2).sum()
    return {
        "layout": f"SBHD [{L}, {B}, {x.H}, {x.D}] bf16, key-padding mask, causal",
        "ms": round(ms, 4),
        "useful_tflops": round(x.flops / (ms * 1e-3) / 1e12, 2),
        "speedup_of_varlen": None,
        "computed_pairs_ratio": round(padded_pairs / real_pairs, 2),
        "samples_timed": timed,
        "extrapolated": timed < B,
    }


def no_isolation_baseline(torch, pvc, x, window=4096, reps=5):
    """The same buffer attended causally per whole window, ignoring document
    boundaries ([opworld] "pitfall one": a 4k window of ten documents wastes
    about 90% of its causal pairs on cross-document attention)."""
    T = x.T
    cu = torch.arange(0, T + 1, window, dtype=torch.int32, device="cuda")
    if int(cu[-1]) != T:
        return None
    ws = torch.empty(pvc.attn_workspace_size(T, cu.numel() - 1), dtype=torch.uint8, device="cuda")
    plan = pvc.AttnPlan(cu, T, window, True, workspace=ws)
    out = torch.empty_like(x.q)
    pvc.varlen_attn_fwd(x.q, x.k, x.v, plan=plan, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        pvc.varlen_attn_fwd(x.q, x.k, x.v, plan=plan, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    pairs = (T // window) * window * (window + 1) / 2
    real = x.w.real_lengths.astype(np.float64)
    return {"layout": f"THD, causal over whole {window}-token windows (documents not isolated)",
            "ms": round(ms, 4), "computed_pairs_ratio": round(pairs / (real * (real + 1) / 2).sum(), 2)}


def measured_peaks(torch):
    """What this GPU sustains on plain library work: a device copy (read +
    write bytes) and a large bf16 GEMM (hipBLASLt through torch)."""
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * n * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    # hipBLASLt through torch: both operands row-major ("nn") and the second
    # one transposed ("nt", x @ y^T), after about 0.4 s of GEMM load (the
    # clock settles under sustained MFMA work); the faster layout is the peak
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(500):
        torch.matmul(x, y)
    torch.cuda.synchronize()
    rates = {}
    for name, rhs in (("nn", y), ("nt", y.t())):
        for _ in range(5):
            torch.matmul(x, rhs)
        torch.cuda.synchronize()
        a.record()
        for _ in range(20):
            torch.matmul(x, rhs)
        b.record()
        torch.cuda.synchronize()
        rates[name] = round(2.0 * m ** 3 * 20 / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    del x, y
    torch.cuda.empty_cache()
    return {"copy_gbps": round(copy_gbps, 1), "copy_bytes": 2 * n,
            "gemm_bf16_tflops": max(rates.values()), "gemm_bf16_tflops_by_layout": rates,
            "gemm_shape": [m, m, m]}


def pack_build_large(torch, pvc, T=1 << 28, reps=5):
    """pack_build at 2^28 tokens with the short-segment length recipe
    (uniform [8, 128]): large enough to be bound by HBM, not by launches."""
    rng = np.random.default_rng([99, 0])
    L = rng.integers(8, 129, size=int(T / 68 * 1.05) + 16).astype(np.int64)
    c = np.cumsum(L)
    n = int(np.searchsorted(c, T))
    L = L[: n + 1].copy()
    L[n] -= int(c[n] - T)
    if L[n] == 0:
        L = L[:n]
    lengths = torch.from_numpy(L.astype(np.int32)).cuda()
    tokens = torch.randint(3, 32000, (T,), dtype=torch.int32, device="cuda")
    pvc.pack_build(lengths, tokens)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        pvc.pack_build(lengths, tokens)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nseg = int(lengths.numel())
    del lengths, tokens
    torch.cuda.empty_cache()
    return {"total_tokens": T, "segments": nseg, "ms": round(ms, 3),
            "gbps": round(pack_bytes(T, nseg) / (ms * 1e-3) / 1e9, 1)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows(w, q, k, v, rows, threads):
    """Time the fp64 attention oracle on query ``rows`` of workload ``w``;
    returns (seconds, useful FLOPs of those rows over all heads of q)."""
    from oracle import attention as A
    from oracle import pack as P
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    pos = P.positions_from_cu(cu)
    t0 = time.perf_counter()
    A.attention_rows(q, k, v, cu, rows, True, threads=threads)
    dt = time.perf_counter() - t0
    return dt, 4.0 * w.head_dim * q.shape[1] * float((pos[rows] + 1).sum())


def cpu_baseline(x, seconds=12.0):
    """The fp64 oracle on a bounded, seeded sample of query rows of the same
    workload, on every host thread this process may use.

    Only the attention oracle is timed (it is the step's cost on the CPU too);
    it runs on the workload's bf16 q/k/v as generated, since the arithmetic
    per row does not depend on the values."""
    from oracle import attention as A
    from oracle import pack as P

    w = x.w
    threads = len(os.sched_getaffinity(0))
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    pos = P.positions_from_cu(cu)
    seg_pad = np.repeat(w.is_pad, w.lengths)
    real_rows = np.nonzero(seg_pad == 0)[0]
    q, k, v = x.host_qkv if x.host_qkv is not None else w.qkv()
    rng = np.random.default_rng(99)
    # calibrate on a small sample, then run seeded batches of random rows
    # until about `seconds` of oracle time has been spent
    probe = rng.choice(real_rows, size=min(256, real_rows.size), replace=False)
    t0 = time.perf_counter()
    A.attention_rows(q, k, v, cu, probe, True, threads=threads)
    rate = probe.size / max(time.perf_counter() - t0, 1e-3)          # rows per second
    n_rows, flops, dt = 0, 0.0, 0.0
    for _ in range(4):
        left = seconds - dt
        if left <= 0.1 * seconds:
            break
        n = int(min(real_rows.size, max(256, rate * left)))
        rows = rng.choice(real_rows, size=n, replace=False)
        t0 = time.perf_counter()
        A.attention_rows(q, k, v, cu, rows, True, threads=threads)
        t = time.perf_counter() - t0
        dt += t
        n_rows += n
        flops += 4.0 * w.head_dim * w.heads * (pos[rows] + 1).sum()
        rate = n / max(t, 1e-3)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_rows} random real query rows x {w.heads} heads of the {w.name} workload, "
                  f"fp64 attention oracle (C loop, {threads} threads, {dt:.1f} s)",
        "seconds": round(dt, 2),
        "cpu": _cpu_model(),
        "host": platform.node(),
    }


def cpu_single_thread():
    """One-thread times of the fp64 attention oracle:
      tiny       the nine-token pack, every row;
      short      the short-segment buffer (65,536 tokens, 16 heads), every row;
      pretrain   the 4k windows, one of 32 heads timed in full (the
                 workload's lengths, one head of N(0,1) bf16 q/k/v), the time
                 scaled by 32 (labelled extrapolated);
      longctx    the long-context buffer, 512 random real rows of one head,
                 the time scaled by useful FLOPs to every row and 32 heads
                 (labelled extrapolated)."""
    from workloads import make_workload
    res = {}
    rng = np.random.default_rng(7)
    for name, heads, sample_rows in (("tiny", None, None), ("short", None, None), ("pretrain", 1, None),
                                     ("longctx", 1, 512)):
        w_full = make_workload(name)
        w = make_workload(name, heads=heads) if heads is not None else w_full
        q, k, v = w.qkv()
        if sample_rows is None:
            rows = np.arange(w.total_tokens, dtype=np.int64)
        else:
            real = np.nonzero(np.repeat(w.is_pad, w.lengths) == 0)[0]
            rows = np.sort(rng.choice(real, size=sample_rows, replace=False))
        dt, fl = _oracle_rows(w, q, k, v, rows, 1)
        total = useful_flops(w_full.lengths, w_full.is_pad, w_full.heads, w_full.head_dim)
        ext = dt * total / fl
        entry = {"seconds_timed": round(dt, 3), "flops_timed": fl, "full_workload_flops": total,
                 "full_workload_seconds": round(ext, 2), "extrapolated": bool(fl < total * 0.999),
                 "tflops": round(fl / dt / 1e12, 5)}
        if heads is not None:
            entry["timed"] = (f"{'all' if sample_rows is None else sample_rows} rows of 1 of "
                              f"{w_full.heads} heads, scaled by useful FLOPs")
        else:
            entry["timed"] = "every row and head"
        res[name] = entry
        del q, k, v
    return {"threads": 1, "cpu": _cpu_model(), "workloads": res}


def roofline(x, attn_ms, kernel, traffic=None):
    """The forward kernel against its binding roof: HBM when the compulsory
    bytes (q, k, v read, o written) at 8 TB/s take longer than the useful
    FLOPs at the bf16 MFMA peak, else MFMA."""
    a_bytes = attn_bytes(x.T, x.H, x.D)
    ai = x.flops / a_bytes
    hbm_roof = ai * PEAK_HBM_GBPS / 1e3
    tflops = x.flops / (attn_ms * 1e-3) / 1e12
    if hbm_roof < PEAK_BF16_TFLOPS:
        bound, achieved, peak, unit, alg = "hbm", a_bytes / (attn_ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s", a_bytes
    else:
        bound, achieved, peak, unit, alg = "mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s", x.flops
    return {
        "kernel": kernel,
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "traffic_unit": "HBM bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0, copy-calibrated)",
        "traffic_over_algorithmic_bytes": None if traffic is None else round(traffic / a_bytes, 3),
        "algorithmic_per_launch": alg,
        "algorithmic_bytes_per_launch": a_bytes,
        "launch_ms": round(attn_ms, 4),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "hbm_roofline_tflops": round(min(hbm_roof, PEAK_BF16_TFLOPS), 1),
        "frac_of_binding_roof_tflops": round(tflops / min(hbm_roof, PEAK_BF16_TFLOPS), 4),
    }


def workload_block(torch, pvc, x, steps, warmup):
    """Step and per-kernel figures of one workload, with its forward roofline."""
    ms_step, stage_ms = time_steps(torch, pvc, x, steps, warmup)
    pack_ms, rope_ms, plan_ms, attn_ms = (float(v) for v in stage_ms)
    tf = x.flops / (attn_ms * 1e-3) / 1e12
    kernel = f"attn_fwd_kernel<{x.D}, causal, bf16 out>"
    return {
        "T": x.T, "real_tokens": x.real_tokens, "segments": x.w.nseg, "pad_segments": int(x.w.is_pad.sum()),
        "max_seqlen": x.max_seqlen, "heads": x.H, "head_dim": x.D,
        "step_ms": round(ms_step, 4),
        "step_useful_tflops": round(x.flops / (ms_step * 1e-3) / 1e12, 2),
        "effective_tokens_per_s": round(x.real_tokens / (ms_step * 1e-3), 1),
        "kernels": {
            "pack_build": {"ms": round(pack_ms, 4),
                           "gbps": round(pack_bytes(x.T, x.w.nseg) / (pack_ms * 1e-3) / 1e9, 1)},
            "rope_thd_apply": {"ms": round(rope_ms, 4),
                               "gbps": round(rope_bytes(x.T, x.H, x.D) / (rope_ms * 1e-3) / 1e9, 1)},
            "attn_plan": {"ms": round(plan_ms, 4)},
            "varlen_attn_fwd": {"ms": round(attn_ms, 4), "useful_tflops": round(tf, 2),
                                "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                                "compulsory_gbps": round(attn_bytes(x.T, x.H, x.D) / (attn_ms * 1e-3) / 1e9, 1),
                                "arith_intensity": round(x.flops / attn_bytes(x.T, x.H, x.D), 1)},
        },
        "roofline": roofline(x, attn_ms, kernel, counter_traffic(x.w.name)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before the timed ones.  A fresh process needs about 30 ms
    # of attention load before the forward reaches its sustained rate: 5 steps
    # of the long-context buffer are 60 ms; the SFT packs need about 50.
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="longctx")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip padded baseline and other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (HBM counter calibration)")
    ap.add_argument("--only", choices=("pack_build_2^28", "prefill"),
                    help="only time one side measurement (for kernel traces and counters) and print it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "reps": 5}), flush=True)
        return
    import packed_varlen_causal_amd as pvc

    if args.only == "pack_build_2^28":
        print(json.dumps({"pack_build_2^28": pack_build_large(torch, pvc, reps=args.steps)}), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps({"prefill": time_prefill(torch, pvc, args.steps, args.warmup)}), flush=True)
        return

    x = Inputs(args.workload, torch, pvc, keep_host=not args.no_cpu_baseline)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    resident = torch.cuda.memory_allocated()
    head = workload_block(torch, pvc, x, args.steps, args.warmup)
    mem_peak = torch.cuda.max_memory_allocated()
    ms_step = head["step_ms"]
    value = x.flops / (ms_step * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": x.w.name, "description": x.w.note, "total_tokens": x.T,
            "real_tokens": x.real_tokens, "segments": x.w.nseg, "pad_segments": int(x.w.is_pad.sum()),
            "max_seqlen": x.max_seqlen, "heads": x.H, "head_dim": x.D, "causal": True,
            "step": "pack_build + rope_thd_apply(q,k) + attn_plan + varlen_attn_fwd",
        },
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "effective_tokens_per_s": head["effective_tokens_per_s"],
        "device_memory": {
            "resident_inputs_and_buffers_bytes": int(resident),
            "peak_during_steps_bytes": int(mem_peak),
            "note": "q, k, v, rotated q and k, output, plan workspace and packing outputs (PyTorch allocator)",
        },
        "kernels": head["kernels"],
        "roofline": head["roofline"],
    }
    attn_ms = head["kernels"]["varlen_attn_fwd"]["ms"]
    attn_tflops = head["kernels"]["varlen_attn_fwd"]["useful_tflops"]
    torch.cuda.synchronize()
    res["kernels"]["varlen_attn_bwd"] = time_backward(torch, pvc, x, max(3, args.steps // 2), BWD_WARMUP)
    res["kernels"]["packed_ce_loss"] = time_ce(torch, pvc, x, max(3, args.steps // 2), 2)

    if not args.no_extras:
        res["padded_sbhd"] = padded_baseline(torch, pvc, x)
        res["padded_sbhd"]["speedup_of_varlen"] = round(res["padded_sbhd"]["ms"] / attn_ms, 2)
        res["measured_peaks"] = measured_peaks(torch)
        res["roofline"]["frac_of_measured_copy"] = round(
            attn_bytes(x.T, x.H, x.D) / (attn_ms * 1e-3) / 1e9 / res["measured_peaks"]["copy_gbps"], 4)
        res["roofline"]["frac_of_measured_gemm"] = round(attn_tflops / res["measured_peaks"]["gemm_bf16_tflops"], 4)
        res["pack_build_2^28"] = pack_build_large(torch, pvc)
        others = {}
        for name in ("sft", "pretrain", "longctx", "short"):
            if name == x.w.name:
                continue
            y = Inputs(name, torch, pvc)
            # the SFT packs and short segments are light: 50 untimed steps
            # bring the clock to its sustained rate (see --warmup)
            blk = workload_block(torch, pvc, y, max(3, args.steps // 2), max(args.warmup, 50))
            blk["backward"] = time_backward(torch, pvc, y, max(3, args.steps // 2), BWD_WARMUP)
            pad = padded_baseline(torch, pvc, y)
            pad["speedup_of_varlen"] = round(pad["ms"] / blk["kernels"]["varlen_attn_fwd"]["ms"], 2)
            blk["padded_sbhd"] = pad
            if name == "pretrain":
                ni = no_isolation_baseline(torch, pvc, y)
                if ni is not None:
                    ni["slowdown_vs_varlen"] = round(ni["ms"] / blk["kernels"]["varlen_attn_fwd"]["ms"], 2)
                    blk["no_isolation"] = ni
            others[name] = blk
            del y
            torch.cuda.empty_cache()
        res["other_workloads"] = others
        res["prefill"] = time_prefill(torch, pvc, max(20, args.steps), max(50, args.warmup))

    if not args.no_cpu_baseline:
        cb = cpu_baseline(x, args.cpu_seconds)
        cb["single_thread"] = cpu_single_thread()
        res["cpu_baseline"] = cb
        res["gpu_over_cpu_oracle"] = round(attn_tflops / cb["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
