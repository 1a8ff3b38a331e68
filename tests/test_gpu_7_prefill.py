"""GPU parity for the prefill path: separate query / key boundaries with the
bottom-right causal alignment, grouped key / value heads (pvc_attn_plan_qk +
pvc_varlen_attn_fwd_qk_planned), against the fp64 oracle attention_qk with the
attention forward's three-part check (fp32 output within 1e-2, bf16 output the
RNE of it, raw bf16 error reported)."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import ATOL, dev_bf16, dev_i32, host_bits, say, three_part_check
from oracle import attention as A
from workloads import f32_to_bf16_bits, make_prefill, prefill_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _bits(shape, seed):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


def _run(pvc, q, k, v, cu_q, cu_k, causal=True):
    cu_q, cu_k = np.asarray(cu_q), np.asarray(cu_k)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    plan = pvc.attn_plan_qk(dev_i32(cu_q), dev_i32(cu_k), q.shape[0], k.shape[0],
                            int(np.diff(cu_q).max()), int(np.diff(cu_k).max()), causal)
    ob = pvc.varlen_attn_fwd_qk(qd, kd, vd, plan=plan, causal=causal)
    of, ls = pvc.varlen_attn_fwd_qk(qd, kd, vd, plan=plan, causal=causal, out_dtype=torch.float32,
                                    return_lse=True)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    return ob, of, ls


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))])


@pytest.mark.parametrize("causal", [True, False])
def test_small_prefill_every_row(pvc, causal):
    pw = make_prefill(scale="small")
    q, k, v = (prefill_bits(pw, x) for x in "qkv")
    cu_q, cu_k = _cu(pw.lq), _cu(pw.lk)
    say(f"  prefill small causal={causal}: Tq={pw.total_q} Tk={pw.total_k} requests={len(pw.lq)} "
        f"H={pw.heads} Hkv={pw.kv_heads}")
    ob, of, ls = _run(pvc, q, k, v, cu_q, cu_k, causal)
    ref, ref_lse = A.attention_qk(q, k, v, cu_q, cu_k, causal)
    three_part_check(of, ob, ref)
    assert np.abs(ls.cpu().numpy().T - ref_lse).max() < 5e-3


@pytest.mark.parametrize("lq,lk,hq,hkv", [
    ([5, 1, 130, 33, 64], [3, 7, 130, 300, 64], 4, 1),    # Lk < Lq, decode, square, long prefix
    ([1] * 40, [200] * 40, 8, 8),                          # forty single-token decodes
    ([257, 2, 129], [257, 2, 129], 6, 3),                  # square requests, grouped heads
    ([300, 17, 128, 1, 90], [500, 17, 300, 40, 90], 16, 4),  # two heads per item-order block
])
def test_edge_requests(pvc, lq, lk, hq, hkv):
    d = 128 if hq % 2 == 0 else 64
    cu_q, cu_k = _cu(lq), _cu(lk)
    say(f"  prefill edge lq={lq[:5]} lk={lk[:5]} H={hq} Hkv={hkv}")
    q = _bits((int(cu_q[-1]), hq, d), 1)
    k, v = _bits((int(cu_k[-1]), hkv, d), 2), _bits((int(cu_k[-1]), hkv, d), 3)
    ob, of, ls = _run(pvc, q, k, v, cu_q, cu_k)
    ref, ref_lse = A.attention_qk(q, k, v, cu_q, cu_k, True)
    three_part_check(of, ob, ref)
    none = np.isneginf(ref_lse[:, 0])
    assert (of.cpu().numpy()[none] == 0).all() and np.isneginf(ls.cpu().numpy().T[none]).all()


def test_square_grouped_equals_repeated_heads_through_the_self_plan(pvc):
    """Square boundaries: the grouped kernel run and the self-attention
    kernel on K/V heads repeated to the query head count both match the
    oracle within the bar, and each other within the same bar.  (They are
    not bit-identical: the grouped run tiles the queries in 32-row tiles,
    the self-attention run in 128-row tiles, so a row's key stages start at
    different offsets and its running max, and with it the bf16 rounding of
    its probabilities, moves at different stages.)"""
    lengths = [100, 37, 300, 64]
    cu = _cu(lengths)
    T = int(cu[-1])
    q, k, v = _bits((T, 8, 128), 4), _bits((T, 2, 128), 5), _bits((T, 2, 128), 6)
    ob, of, _ = _run(pvc, q, k, v, cu, cu)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    qd, krd, vrd = dev_bf16(q), dev_bf16(kr), dev_bf16(vr)
    o_self = pvc.varlen_attn_fwd(qd, krd, vrd, dev_i32(cu), 300, out_dtype=torch.float32)
    ob_self = pvc.varlen_attn_fwd(qd, krd, vrd, dev_i32(cu), 300)
    torch.cuda.synchronize()
    ref, _ = A.attention_qk(q, k, v, cu, cu, True)
    three_part_check(of, ob, ref)
    three_part_check(o_self, ob_self, ref)
    assert (of - o_self).abs().max().item() <= ATOL


def test_full_size_sampled_rows(pvc):
    pw = make_prefill()
    q, k, v = (prefill_bits(pw, x) for x in "qkv")
    cu_q, cu_k = _cu(pw.lq), _cu(pw.lk)
    say(f"  prefill full: Tq={pw.total_q} Tk={pw.total_k} requests={len(pw.lq)}")
    ob, of, _ = _run(pvc, q, k, v, cu_q, cu_k)
    rows = np.unique(np.concatenate([cu_q[:-1], cu_q[1:] - 1, np.random.default_rng(0).integers(0, pw.total_q, 150)]))
    ref, _ = A.attention_qk(q, k, v, cu_q, cu_k, True, rows=rows)
    three_part_check(of, ob, ref[rows], rows=rows)


def test_plans_are_not_interchangeable(pvc):
    """A prefill plan given to the self-attention forward (and a self plan to
    the prefill forward) sets PVC_DEV_PLAN and writes nothing."""
    cu = dev_i32([0, 30, 64])
    T, H, d = 64, 2, 64
    q, k, v = (dev_bf16(_bits((T, H, d), s)) for s in (1, 2, 3))
    qk = pvc.attn_plan_qk(cu, cu, T, T, 34, 34, True)
    out = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    st = pvc._lib.pvc_varlen_attn_fwd_planned(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), None, T, H, d, 1, 0, ctypes.c_void_p(qk.workspace.data_ptr()),
        qk.ws_bytes, ctypes.c_void_p(qk.dev_error.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and int(qk.dev_error.item()) & 128 and (out.float() == 7.0).all()
    selfp = pvc.attn_plan(cu, T, 34, True)
    out2 = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    st = pvc._lib.pvc_varlen_attn_fwd_qk_planned(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out2.data_ptr()), None, T, T, H, H, d, 1, 0, ctypes.c_void_p(selfp.workspace.data_ptr()),
        selfp.ws_bytes, ctypes.c_void_p(selfp.dev_error.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and int(selfp.dev_error.item()) & 128 and (out2.float() == 7.0).all()


@pytest.mark.parametrize("cu_q,Tq", [([-300, 40, 64], 64), ([-1000, -500, 300], 300)])
def test_malformed_query_boundaries_write_nothing(pvc, cu_q, Tq):
    """A cu_seqlens_q with a negative first entry: the plan clamps the query
    ranges it decodes the tile order from (an unclamped range once gave tile
    -1), flags PVC_DEV_CU0 and the forward writes nothing."""
    cu_k = [0, 30, 64]
    H, d = 16, 128
    say(f"  prefill malformed cu_q={cu_q} Tq={Tq}")
    q = dev_bf16(_bits((Tq, H, d), 1))
    k, v = dev_bf16(_bits((64, 4, d), 2)), dev_bf16(_bits((64, 4, d), 3))
    plan = pvc.attn_plan_qk(dev_i32(cu_q), dev_i32(cu_k), Tq, 64, Tq, 64, True)
    out = torch.full((Tq, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    pvc.varlen_attn_fwd_qk(q, k, v, plan=plan, out=out)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) & 1
    assert (out.float() == 7.0).all()


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, False)])
def test_four_query_heads_per_kv_head_every_row(pvc, d, causal):
    """Groups of 4 (and 8) query heads per key / value head run four query
    heads per workgroup on 32-row tiles; every row against the oracle,
    including requests shorter than a tile and rows with no visible key."""
    lq = [1, 31, 32, 33, 100, 7, 64, 5]
    lk = [40, 31, 32, 60, 100, 3, 200, 9]
    cu_q, cu_k = _cu(lq), _cu(lk)
    for hq, hkv in ((8, 2), (8, 1)):
        say(f"  prefill grouped d={d} causal={causal} H={hq} Hkv={hkv}")
        q = _bits((int(cu_q[-1]), hq, d), 11)
        k, v = _bits((int(cu_k[-1]), hkv, d), 12), _bits((int(cu_k[-1]), hkv, d), 13)
        ob, of, ls = _run(pvc, q, k, v, cu_q, cu_k, causal)
        ref, ref_lse = A.attention_qk(q, k, v, cu_q, cu_k, causal)
        three_part_check(of, ob, ref)
        fin = np.isfinite(ref_lse)
        assert np.abs(ls.cpu().numpy().T[fin] - ref_lse[fin]).max() < 5e-3
        assert np.isneginf(ls.cpu().numpy().T[~fin]).all()


def _align(x, a=256):
    return (x + a - 1) // a * a


def _plan_tile_order(plan):
    """The plan's tile-order table: the workspace holds a 256-byte header, the
    per-row key ranges and query segments (int2 per query row each, every
    region 256-byte aligned), then one int32 per 32-row query tile."""
    T = plan.total_q
    off = 256 + 2 * _align(8 * T)
    nt = (T + 31) // 32
    return plan.workspace[off:off + 4 * nt].cpu().numpy().view(np.int32).copy()


def _expected_tile_order(cu_q, cu_k, causal, chunk=16, max_chunks=2048):
    """The start order of the 32-row tiles, written from its definition: a
    tile belongs to the request of its first row; each request's tiles are cut
    into chunks of 16 from its last tile down; chunks go in decreasing order of
    the key span of their heaviest tile (first row's range start to last
    row's range end), ties by the chunk's last tile; more than 2048 chunks:
    requests in buffer order, each request's tiles last to first."""
    cu_q, cu_k = np.asarray(cu_q, np.int64), np.asarray(cu_k, np.int64)
    Tq = int(cu_q[-1])
    nt = (Tq + 31) // 32
    x = np.zeros(Tq, np.int64)
    y = np.zeros(Tq, np.int64)
    for r in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[r], cu_q[r + 1], cu_k[r], cu_k[r + 1]
        i = np.arange(qs, qe)
        n = np.minimum(ke - ks, i - qs + (ke - ks) - (qe - qs) + 1) if causal else np.full(i.size, ke - ks)
        x[i] = ks
        y[i] = ks + np.maximum(n, 0)
    span = [max(int(y[min(32 * t + 31, Tq - 1)] - x[32 * t]), 0) for t in range(nt)]
    chunks = []
    for r in range(len(cu_q) - 1):
        ta, tb = -(-int(cu_q[r]) // 32), -(-int(cu_q[r + 1]) // 32)
        for hi in range(tb, ta, -chunk):
            lo = max(ta, hi - chunk)
            chunks.append((hi, hi - lo, max(span[lo:hi])))
    if len(chunks) > max_chunks:
        order = []
        for r in range(len(cu_q) - 1):
            ta, tb = -(-int(cu_q[r]) // 32), -(-int(cu_q[r + 1]) // 32)
            order += list(range(tb - 1, ta - 1, -1))
        return np.asarray(order, np.int32)
    chunks.sort(key=lambda c: (-c[2], c[0]))
    return np.asarray([hi - 1 - i for hi, n, _ in chunks for i in range(n)], np.int32)


@pytest.mark.parametrize("which,causal", [("prefill", True), ("prefill", False), ("many_short", True)])
def test_tile_order_is_the_sorted_chunk_permutation(pvc, which, causal):
    """The plan's tile order equals the one written from its definition (the
    full prefill, causal and not: sorted chunks; 3,000 short requests: more
    than 2,048 chunks, the buffer order), so every tile is run exactly once."""
    if which == "prefill":
        pw = make_prefill()
        lq, lk = pw.lq, pw.lk
    else:
        rng = np.random.default_rng(5)
        lq = rng.integers(20, 45, size=3000)
        lk = lq + rng.integers(0, 100, size=3000)
    cu_q, cu_k = _cu(lq), _cu(lk)
    say(f"  tile order {which} causal={causal}: Tq={int(cu_q[-1])} requests={len(lq)}")
    plan = pvc.attn_plan_qk(dev_i32(cu_q), dev_i32(cu_k), int(cu_q[-1]), int(cu_k[-1]), int(np.max(lq)),
                            int(np.max(lk)), causal)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    got = _plan_tile_order(plan)
    want = _expected_tile_order(cu_q, cu_k, causal)
    nt = (int(cu_q[-1]) + 31) // 32
    assert np.array_equal(np.sort(got), np.arange(nt))
    assert np.array_equal(got, want)


def test_full_prefill_writes_every_row(pvc):
    """Every query row of the full prefill is written (output prefilled with
    NaN), in the launch the bench times."""
    pw = make_prefill()
    cu_q, cu_k = _cu(pw.lq), _cu(pw.lk)
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.randn((pw.total_q, pw.heads, pw.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((pw.total_k, pw.kv_heads, pw.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn_like(k)
    plan = pvc.attn_plan_qk(dev_i32(cu_q), dev_i32(cu_k), pw.total_q, pw.total_k, int(pw.lq.max()),
                            int(pw.lk.max()), True)
    out = torch.full_like(q, float("nan"))
    say(f"  prefill full coverage Tq={pw.total_q} Tk={pw.total_k}")
    pvc.varlen_attn_fwd_qk(q, k, v, plan=plan, out=out)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    assert not torch.isnan(out.float()).any()
