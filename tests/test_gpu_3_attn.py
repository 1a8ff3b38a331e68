"""GPU parity for the varlen attention forward (and the padded-SBHD baseline).

Against the fp64 oracle with the three-part check in gpu_util: the kernel's
fp32 output within 1e-2 max-abs, its bf16 output equal to the RNE rounding of
that fp32 output, raw bf16 error reported.  Exact cases from the pages are
checked bit for bit on the bf16 product path.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_util import ATOL, dev_bf16, dev_i32, host_bits, say, three_part_check
from oracle import attention as A
from oracle import pack as P
from workloads import CONFIG_NAMES, f32_to_bf16_bits, make_workload, qkv_bits

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _rand_bits(shape, seed, scale=1.0):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale)


def _run(pvc, q, k, v, cu, causal=True, max_seqlen=None, lse=False):
    """Both output modes on the same plan; returns (bf16 out, fp32 out[, lse])."""
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    cu = np.asarray(cu)
    mx = int((cu[1:] - cu[:-1]).max()) if max_seqlen is None else max_seqlen
    plan = pvc.attn_plan(dev_i32(cu), q.shape[0], mx, causal)
    ob = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal)
    of, ls = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, out_dtype=torch.float32,
                                 return_lse=True)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    return ob, of, ls


def test_zero_score_example(pvc, golden):
    """All scores zero; V = 1 on A, 10 on b0: b0 outputs 10 isolated, 3.25 whole-pack."""
    case = golden("attention_examples.json")["zero_score"]
    T, H, d = 9, 2, 64
    q = f32_to_bf16_bits(np.zeros((T, H, d), np.float32))
    k = _rand_bits((T, H, d), 1)
    vf = np.random.default_rng(2).standard_normal((T, H, d)).astype(np.float32)
    vf[0:3] = case["v_A"]
    vf[3] = case["v_b0"]
    v = f32_to_bf16_bits(vf)
    say("  attn zero-score example")
    ob, of, _ = _run(pvc, q, k, v, [0, 3, 5, 9])
    assert (ob.float().cpu()[3] == case["expected_b0_isolated"]).all()
    ob, of, _ = _run(pvc, q, k, v, [0, 9])
    assert (ob.float().cpu()[3] == case["expected_b0_whole_pack"]).all()
    assert (of.cpu()[3] == case["expected_b0_whole_pack"]).all()


def test_zero_score_through_whole_path(pvc, golden):
    """pack_build -> RoPE -> attention on the nine-token pack (q = 0 stays 0 under RoPE)."""
    case = golden("attention_examples.json")["zero_score"]
    w = make_workload("tiny")
    q = f32_to_bf16_bits(np.zeros((9, w.heads, w.head_dim), np.float32))
    k = qkv_bits(w, "k")
    vf = np.zeros((9, w.heads, w.head_dim), np.float32)
    vf[0:3], vf[3] = case["v_A"], case["v_b0"]
    meta = pvc.pack_build(dev_i32(w.lengths), dev_i32(w.tokens()))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(f32_to_bf16_bits(vf))
    pvc.rope_thd_apply(qd, kd, meta["cu_seqlens"], w.rope_base)
    out = pvc.varlen_attn_fwd(qd, kd, vd, meta["cu_seqlens"], int(w.lengths.max()))
    torch.cuda.synchronize()
    assert (out.float().cpu()[3] == case["expected_b0_isolated"]).all()


@pytest.mark.parametrize("name", CONFIG_NAMES)
@pytest.mark.parametrize("causal", [True, False])
def test_small_workloads_every_element(pvc, name, causal):
    w = make_workload(name, scale="small")
    say(f"  attn small {name} causal={causal}: T={w.total_tokens} nseg={w.nseg} H={w.heads} d={w.head_dim}")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    ob, of, ls = _run(pvc, q, k, v, cu, causal)
    ref, ref_lse = A.attention(q, k, v, cu, causal, threads=THREADS)
    three_part_check(of, ob, ref)
    lse_err = np.abs(ls.cpu().numpy().T - ref_lse).max()
    say(f"    lse max abs {lse_err:.2e}")
    assert lse_err < 5e-3


@pytest.mark.parametrize("heads", [16, 24])
@pytest.mark.parametrize("causal", [True, False])
def test_head_counts_divisible_by_the_xcds(pvc, heads, causal):
    """Head counts that are multiples of 8 take the item order that
    interleaves a block of heads inside each segment's run of tiles (2 and 3
    heads per block here): every element of every head against the oracle."""
    lengths = np.array([700, 3, 129, 1, 250, 512, 64, 1200, 33])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, d = int(cu[-1]), 128
    say(f"  head blocks: H={heads} causal={causal} T={T}")
    q, k, v = (_rand_bits((T, heads, d), s) for s in (31, 32, 33))
    ob, of, ls = _run(pvc, q, k, v, cu, causal)
    ref, ref_lse = A.attention(q, k, v, cu, causal, threads=THREADS)
    three_part_check(of, ob, ref)
    assert np.abs(ls.cpu().numpy().T - ref_lse).max() < 5e-3


def test_more_segments_than_the_fused_plan_launch(pvc):
    """Beyond 16,384 segments the plan's check runs as its own launch: the
    same results on 20,000 short segments (sampled rows against the oracle,
    every segment boundary included among them)."""
    lengths = np.random.default_rng(7).integers(1, 9, 20000)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(cu[-1]), 2, 64
    say(f"  many segments: nseg={lengths.size} T={T}")
    q, k, v = (_rand_bits((T, H, d), s) for s in (51, 52, 53))
    ob, of, ls = _run(pvc, q, k, v, cu, True)
    rows = np.unique(np.concatenate([cu[:-1][::37], cu[1:][::41] - 1,
                                     np.random.default_rng(8).integers(0, T, 300)]))
    ref, ref_lse = A.attention_rows(q, k, v, cu, rows, True, threads=THREADS)
    three_part_check(of, ob, ref, rows=rows)
    assert np.abs(ls.cpu().numpy().T[rows] - ref_lse).max() < 5e-3


@pytest.mark.parametrize("lengths", [[1], [1] * 200, [1000], [130, 1, 127, 300, 2, 64, 65],
                                     [33, 31, 32, 64, 96, 129], [4096 + 17]])
def test_edge_lengths(pvc, lengths):
    T = sum(lengths)
    H, d = 2, 128 if T % 2 else 64
    say(f"  attn edge lengths n={len(lengths)} T={T} d={d}")
    q, k, v = (_rand_bits((T, H, d), s) for s in (1, 2, 3))
    cu = P.pack_build(lengths)["cu_seqlens"]
    ob, of, _ = _run(pvc, q, k, v, cu)
    rows = np.arange(T) if T <= 2000 else np.unique(np.concatenate([np.arange(0, T, 7), [T - 1]]))
    ref, _ = A.attention_rows(q, k, v, cu, rows, True, threads=THREADS)
    three_part_check(of, ob, ref, rows=rows)


def test_max_seqlen_larger_than_actual_is_accepted(pvc):
    lengths = [40, 7, 90]
    T = sum(lengths)
    q, k, v = (_rand_bits((T, 2, 64), s) for s in (4, 5, 6))
    cu = P.pack_build(lengths)["cu_seqlens"]
    ob, of, _ = _run(pvc, q, k, v, cu, max_seqlen=4096)
    three_part_check(of, ob, A.attention(q, k, v, cu)[0])


def test_single_key_rows_and_constant_v_exact(pvc):
    w = make_workload("short", scale="small")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    ob, _, _ = _run(pvc, q, k, v, cu)
    starts = cu[:-1]
    assert (host_bits(ob)[starts] == v[starts]).all()       # one visible key: o = v exactly
    vc = f32_to_bf16_bits(np.full(v.shape, -2.71875, np.float32))
    ob, _, _ = _run(pvc, q, k, vc, cu)
    assert (host_bits(ob) == vc).all()                        # constant V: o = c exactly


def test_changing_one_segment_leaves_others_bit_identical(pvc):
    w = make_workload("sft", scale="small")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    ob1, of1, _ = _run(pvc, q, k, v, cu)
    r = 3
    s, e = int(cu[r]), int(cu[r + 1])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x, seed in ((q2, 7), (k2, 8), (v2, 9)):
        x[s:e] = _rand_bits(x[s:e].shape, seed, 3.0)
    ob2, of2, _ = _run(pvc, q2, k2, v2, cu)
    b1, b2 = host_bits(ob1), host_bits(ob2)
    keep = np.ones(w.total_tokens, bool)
    keep[s:e] = False
    assert (b1[keep] == b2[keep]).all()
    assert (of1.cpu().numpy()[keep] == of2.cpu().numpy()[keep]).all()
    assert (b1[s:e] != b2[s:e]).any()


def test_packed_matches_each_segment_alone(pvc):
    w = make_workload("longctx", scale="small")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    _, of, _ = _run(pvc, q, k, v, cu)
    packed = of.cpu().numpy()
    for r in range(w.nseg):
        s, e = int(cu[r]), int(cu[r + 1])
        _, alone, _ = _run(pvc, q[s:e], k[s:e], v[s:e], [0, e - s])
        diff = np.abs(alone.cpu().numpy() - packed[s:e]).max()
        assert diff <= ATOL, (r, diff)


def test_deterministic_and_plan_reuse(pvc):
    w = make_workload("pretrain", scale="small")
    q, k, v = w.qkv()
    cu = dev_i32(P.pack_build(w.lengths)["cu_seqlens"])
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    plan = pvc.attn_plan(cu, w.total_tokens, 400)
    outs = [host_bits(pvc.varlen_attn_fwd(qd, kd, vd, plan=plan)) for _ in range(3)]
    fresh = host_bits(pvc.varlen_attn_fwd(qd, kd, vd, cu, 400))
    for o in outs[1:] + [fresh]:
        assert (o == outs[0]).all()


@pytest.mark.parametrize("name", ["sft", "pretrain", "longctx", "short"])
def test_full_size_sampled_rows(pvc, name):
    """The launch configuration the benchmark times, checked on sampled rows."""
    w = make_workload(name)
    say(f"  attn full {name}: T={w.total_tokens} nseg={w.nseg} H={w.heads} d={w.head_dim}")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    ob, of, ls = _run(pvc, q, k, v, cu, max_seqlen=int(w.lengths.max()))
    rng = np.random.default_rng(1)
    longest = int(np.argmax(w.lengths))
    tail = np.arange(max(int(cu[longest]), int(cu[longest + 1]) - 4), int(cu[longest + 1]))
    rows = np.unique(np.concatenate([cu[:-1][:64], (cu[1:] - 1)[:64], tail,
                                     rng.integers(0, w.total_tokens, 96)])).astype(np.int64)
    say(f"    oracle on {rows.size} rows x {w.heads} heads ({THREADS} threads)")
    ref, ref_lse = A.attention_rows(q, k, v, cu, rows, True, threads=THREADS)
    three_part_check(of, ob, ref, rows=rows)
    lse_err = np.abs(ls.cpu().numpy().T[rows] - ref_lse).max()
    assert lse_err < 5e-3


def test_invalid_cu_writes_nothing_and_sets_bits(pvc):
    T, H, d = 9, 2, 64
    q, k, v = (dev_bf16(_rand_bits((T, H, d), s)) for s in (1, 2, 3))
    for bad, bit in (([0, 3, 3, 9], P.ERR_NOT_INCREASING), ([1, 3, 5, 9], P.ERR_CU0),
                     ([0, 3, 5, 8], P.ERR_TOTAL), ([0, 3, 5, 9, 4], P.ERR_NOT_INCREASING)):
        plan = pvc.attn_plan(dev_i32(bad), T, 16)
        out = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
        pvc.varlen_attn_fwd(q, k, v, plan=plan, out=out)
        torch.cuda.synchronize()
        assert int(plan.dev_error.item()) & bit, bad
        assert (out.float() == 7.0).all()


def test_plan_for_other_arguments_is_refused(pvc):
    T, H, d = 64, 2, 64
    q, k, v = (dev_bf16(_rand_bits((T, H, d), s)) for s in (1, 2, 3))
    plan = pvc.attn_plan(dev_i32([0, 30, 64]), T, 34, causal=True)
    out = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lib = pvc._lib
    st = lib.pvc_varlen_attn_fwd_planned(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), None, T, H, d, 0, 0, ctypes.c_void_p(plan.workspace.data_ptr()),
        plan.ws_bytes, ctypes.c_void_p(plan.dev_error.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert int(plan.dev_error.item()) & 128
    assert (out.float() == 7.0).all()


@pytest.mark.parametrize("d,causal", [(64, True), (128, True), (128, False)])
def test_padded_sbhd_baseline(pvc, d, causal):
    """Valid rows of the padded layout equal per-sample attention (the oracle)."""
    lengths = [70, 5, 128, 1, 33]
    L, B, H = 128, len(lengths), 2
    q, k, v = (_rand_bits((L, B, H, d), s) for s in (11, 12, 13))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    sl = dev_i32(lengths)
    ob = pvc.padded_attn_fwd_sbhd(qd, kd, vd, sl, causal)
    of = pvc.padded_attn_fwd_sbhd(qd, kd, vd, sl, causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(of).all()
    for b, n in enumerate(lengths):
        ref, _ = A.attention(q[:n, b], k[:n, b], v[:n, b], [0, n], causal)
        three_part_check(of[:n, b], ob[:n, b], ref)
