"""GPU parity for the varlen attention backward (dQ, dK, dV from the saved LSE).

The kernels take the forward's bf16 output and fp32 log-sum-exp.  Their fp32
gradients are compared with the fp64 oracle (oracle.attention.attention_bwd)
element by element within the first-order bound of gpu_util.grad_error_bounds,
and the bf16 gradients must equal the RNE rounding of the fp32 ones bit for bit
(the two modes differ only in the final store).
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_util import dev_bf16, dev_i32, grad_check, grad_error_bounds, host_bits, say
from oracle import attention as A
from oracle import pack as P
from workloads import CONFIG_NAMES, f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _rand_bits(shape, seed, scale=1.0):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale)


def _fwd_bwd(pvc, q, k, v, g, cu, causal=True):
    """Forward (bf16 out + lse), then the backward in both gradient dtypes."""
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, g))
    cu = np.asarray(cu)
    mx = int((cu[1:] - cu[:-1]).max())
    plan = pvc.attn_plan(dev_i32(cu), q.shape[0], mx, causal)
    out, lse = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, return_lse=True)
    g32 = pvc.varlen_attn_bwd(qd, kd, vd, out, gd, lse, plan, causal, grad_dtype=torch.float32)
    g16 = pvc.varlen_attn_bwd(qd, kd, vd, out, gd, lse, plan, causal)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    return g32, g16


def _check(pvc, q, k, v, g, cu, causal=True, heads=None, segments=None, rows=None):
    g32, g16 = _fwd_bwd(pvc, q, k, v, g, cu, causal)
    refs = A.attention_bwd(q, k, v, g, cu, causal, threads=THREADS, heads=heads, segments=segments)
    bounds = grad_error_bounds(q, k, v, g, cu, causal, heads=heads, segments=segments)
    return grad_check(g32, g16, refs, bounds, rows=rows), g32, g16


@pytest.mark.parametrize("name", CONFIG_NAMES)
@pytest.mark.parametrize("causal", [True, False])
def test_small_workloads_every_element(pvc, name, causal):
    w = make_workload(name, scale="small")
    say(f"  bwd small {name} causal={causal}: T={w.total_tokens} nseg={w.nseg} H={w.heads} d={w.head_dim}")
    q, k, v, g = w.qkv("qkvg")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    _check(pvc, q, k, v, g, cu, causal)


@pytest.mark.parametrize("lengths", [[1], [1] * 200, [1000], [130, 1, 127, 300, 2, 64, 65],
                                     [33, 31, 32, 64, 96, 129], [4096 + 17]])
@pytest.mark.parametrize("causal", [True, False])
def test_edge_lengths(pvc, lengths, causal):
    T = sum(lengths)
    H, d = 2, 128 if T % 2 else 64
    say(f"  bwd edge lengths n={len(lengths)} T={T} d={d} causal={causal}")
    q, k, v, g = (_rand_bits((T, H, d), s) for s in (1, 2, 3, 4))
    cu = P.pack_build(lengths)["cu_seqlens"]
    _check(pvc, q, k, v, g, cu, causal)


def test_large_values(pvc):
    """Scores spread over a wide range (q, k scaled by 4): sharp softmax rows."""
    lengths = [700, 300, 57]
    T, H, d = sum(lengths), 2, 128
    say(f"  bwd large values T={T}")
    q, k = _rand_bits((T, H, d), 21, 4.0), _rand_bits((T, H, d), 22, 4.0)
    v, g = _rand_bits((T, H, d), 23), _rand_bits((T, H, d), 24, 3.0)
    cu = P.pack_build(lengths)["cu_seqlens"]
    _check(pvc, q, k, v, g, cu, True)


def test_changing_one_segment_leaves_other_gradients_bit_identical(pvc):
    w = make_workload("sft", scale="small")
    say("  bwd segment isolation")
    q, k, v, g = w.qkv("qkvg")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    g1, _ = _fwd_bwd(pvc, q, k, v, g, cu)
    r = 3
    s, e = int(cu[r]), int(cu[r + 1])
    x = [q.copy(), k.copy(), v.copy(), g.copy()]
    for arr, seed in zip(x, (7, 8, 9, 10)):
        arr[s:e] = _rand_bits(arr[s:e].shape, seed, 2.0)
    g2, _ = _fwd_bwd(pvc, *x, cu)
    keep = np.ones(w.total_tokens, bool)
    keep[s:e] = False
    for t1, t2 in zip(g1, g2):
        a1, a2 = t1.cpu().numpy(), t2.cpu().numpy()
        assert (a1[keep] == a2[keep]).all()
        assert (a1[s:e] != a2[s:e]).any()


def test_deterministic(pvc):
    w = make_workload("pretrain", scale="small")
    say("  bwd determinism")
    q, k, v, g = w.qkv("qkvg")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, g))
    plan = pvc.attn_plan(dev_i32(cu), w.total_tokens, 400)
    out, lse = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, return_lse=True)
    runs = [[host_bits(t) for t in pvc.varlen_attn_bwd(qd, kd, vd, out, gd, lse, plan)] for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert (a == b).all()


def test_scratch_reused_across_calls(pvc):
    """One scratch buffer, filled with 0xFF, serves a large and then a small
    backward.  The dK/dV work counters sit after the lse / D planes, at an
    offset that depends on the call's size, and the dQ launch zeroes them on
    every call: left at 0xFF they would read as a drained queue and no dK / dV
    would be written.  Both calls must match calls with fresh buffers bit for bit."""
    say("  bwd scratch reused across calls")
    cases = []
    for name, seed in (("pretrain", 31), ("sft", 32)):
        w = make_workload(name, scale="small")
        q, k, v, g = (_rand_bits((w.total_tokens, w.heads, w.head_dim), seed + i) for i in range(4))
        cu = P.pack_build(w.lengths)["cu_seqlens"]
        qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, g))
        plan = pvc.attn_plan(dev_i32(cu), w.total_tokens, int(w.lengths.max()))
        out, lse = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, return_lse=True)
        cases.append((w, (qd, kd, vd, out, gd, lse, plan)))
    size = max(pvc.attn_bwd_scratch_size(w.total_tokens, w.heads) for w, _ in cases)
    shared = torch.full((size,), 0xFF, dtype=torch.uint8, device="cuda")
    reused = [[host_bits(t) for t in pvc.varlen_attn_bwd(*args, scratch=shared)] for _, args in cases]
    fresh = [[host_bits(t) for t in pvc.varlen_attn_bwd(*args)] for _, args in cases]
    torch.cuda.synchronize()
    for r, f in zip(reused, fresh):
        for a, b in zip(r, f):
            assert (a == b).all()


def test_explicit_side_stream_with_library_temporaries(pvc):
    """Forward with plan=None and backward with scratch=None, both on an
    explicit stream that is not torch's current one: the plan workspace, the
    error word and the backward scratch are allocated on that stream, so the
    allocator does not hand their memory to the current stream's work (here
    a stream of fills of fresh tensors) while the kernels still read them.
    Results must equal the current-stream calls bit for bit."""
    w = make_workload("sft", scale="small")
    say("  fwd / bwd on a side stream with library temporaries")
    q, k, v, g = (_rand_bits((w.total_tokens, w.heads, w.head_dim), 40 + i) for i in range(4))
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd, vd, gd, cud = (*(dev_bf16(x) for x in (q, k, v, g)), dev_i32(cu))
    mx = int(w.lengths.max())
    out0, lse0 = pvc.varlen_attn_fwd(qd, kd, vd, cud, mx, return_lse=True)
    plan0 = pvc.attn_plan(cud, w.total_tokens, mx)
    grads0 = pvc.varlen_attn_bwd(qd, kd, vd, out0, gd, lse0, plan0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out1, lse1 = pvc.varlen_attn_fwd(qd, kd, vd, cud, mx, return_lse=True, stream=side)
    plan1 = pvc.attn_plan(cud, w.total_tokens, mx, stream=side)
    grads1 = pvc.varlen_attn_bwd(qd, kd, vd, out1, gd, lse1, plan1, stream=side)
    junk = [torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(32)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert int(plan1.dev_error.item()) == 0
    assert (host_bits(out1) == host_bits(out0)).all()
    assert torch.equal(lse1, lse0)
    for a, b in zip(grads1, grads0):
        assert (host_bits(a) == host_bits(b)).all()


@pytest.mark.parametrize("name", ["sft", "pretrain", "longctx", "short"])
def test_full_size_sampled_segments(pvc, name):
    """The benchmark's launch configuration; the oracle on sampled segments and heads."""
    w = make_workload(name)
    q, k, v, g = w.qkv("qkvg")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    L = w.lengths
    # first, last and the longest segment of at most 2048 tokens, plus a few random ones
    rng = np.random.default_rng(3)
    fit = np.flatnonzero(L <= 2048)
    segs = {0, w.nseg - 1, int(fit[np.argmax(L[fit])])} | set(rng.choice(fit, 3, replace=False).tolist())
    segs = sorted(s for s in segs if L[s] <= 2048)
    heads = [0, w.heads - 1]
    say(f"  bwd full {name}: T={w.total_tokens} nseg={w.nseg} H={w.heads} d={w.head_dim}; "
        f"oracle on segments {segs} (lengths {[int(L[s]) for s in segs]}) heads {heads}")
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in segs])
    _check(pvc, q, k, v, g, cu, True, heads=heads, segments=segs, rows=rows)


def test_invalid_plan_writes_nothing(pvc):
    """A plan built for causal attention used non-causally, and a plan of an
    invalid cu_seqlens: the error bits are set and no gradient is written."""
    T, H, d = 64, 2, 64
    q, k, v, g = (dev_bf16(_rand_bits((T, H, d), s)) for s in (1, 2, 3, 4))
    out = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((H, T), dtype=torch.float32, device="cuda")
    lib = pvc._lib
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    for cu, causal_plan, causal_call, bit in (([0, 30, 64], True, 0, 128), ([0, 30, 30, 64], True, 1, P.ERR_NOT_INCREASING)):
        say(f"  bwd invalid plan cu={cu} plan causal={causal_plan} call causal={causal_call}")
        plan = pvc.attn_plan(dev_i32(cu), T, 34, causal=causal_plan)
        grads = [torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        nb = pvc.attn_bwd_scratch_size(T, H)
        scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
        st = lib.pvc_varlen_attn_bwd_planned(
            vp(q), vp(k), vp(v), vp(out), vp(g), vp(lse), *(vp(t) for t in grads), T, H, d, causal_call, 0,
            vp(plan.workspace), plan.ws_bytes, vp(scratch), nb, vp(plan.dev_error),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == 0
        assert int(plan.dev_error.item()) & bit
        for t in grads:
            assert (t.float() == 7.0).all()
