"""GPU parity for padded storage (cu_seqlens_padded): every segment's tokens at
the start of a slot, the rest of the slot padding.

Forward and backward are compared with the fp64 padded-storage oracle
(oracle.attention.attention_padded / attention_bwd_padded) with the same
checks as the unpadded paths; padding rows must come out exactly 0 (LSE -inf,
gradients 0) and their contents must not change any real row.  RoPE with
cu_seqlens_padded counts positions from each slot start: bit-exact against
the oracle on the compact buffer.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev_bf16, dev_i32, grad_check, grad_error_bounds, host_bits, say, three_part_check
from oracle import attention as A
from oracle import rope as R
from workloads import f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _layout(lengths, align):
    lengths = np.asarray(lengths, np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    slots = (lengths + align - 1) // align * align
    cp = np.concatenate([[0], np.cumsum(slots)])
    return cu, cp


def _bits(shape, seed, scale=1.0):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale)


def _fwd(pvc, q, k, v, cu, cp, causal=True):
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    mx = int((cu[1:] - cu[:-1]).max())
    plan = pvc.attn_plan(dev_i32(cu), q.shape[0], mx, causal, cu_seqlens_padded=dev_i32(cp))
    ob = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal)
    of, ls = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) == 0
    return plan, (qd, kd, vd), ob, of, ls


CASES = [("sft", 64), ("short", 16), ("pretrain", 128), ("longctx", 96)]


@pytest.mark.parametrize("name,align", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_forward_small_workloads(pvc, name, align, causal):
    w = make_workload(name, scale="small")
    cu, cp = _layout(w.lengths, align)
    Ts, H, d = int(cp[-1]), w.heads, w.head_dim
    say(f"  padded fwd {name} align={align} causal={causal}: T={w.total_tokens} storage={Ts}")
    q, k, v = (_bits((Ts, H, d), s) for s in (1, 2, 3))
    _, _, ob, of, ls = _fwd(pvc, q, k, v, cu, cp, causal)
    ref, ref_lse = A.attention_padded(q, k, v, cu, cp, causal, threads=16)
    real = A.storage_rows(cu, cp)
    gap = np.setdiff1d(np.arange(Ts), real)
    three_part_check(of, ob, ref[real], rows=real)
    assert (host_bits(ob)[gap] == 0).all() and (of.cpu().numpy()[gap] == 0).all()
    lse = ls.cpu().numpy().T
    assert np.isneginf(lse[gap]).all()
    assert np.abs(lse[real] - ref_lse[real]).max() < 5e-3


def test_forward_sixteen_heads(pvc):
    """16 heads: the item order interleaves two heads per segment run, which
    must also hold for padding rows (runs of one position)."""
    w = make_workload("sft", scale="small")
    cu, cp = _layout(w.lengths, 64)
    Ts, H, d = int(cp[-1]), 16, w.head_dim
    q, k, v = (_bits((Ts, H, d), s) for s in (41, 42, 43))
    _, _, ob, of, ls = _fwd(pvc, q, k, v, cu, cp, True)
    ref, ref_lse = A.attention_padded(q, k, v, cu, cp, True, threads=16)
    real = A.storage_rows(cu, cp)
    gap = np.setdiff1d(np.arange(Ts), real)
    three_part_check(of, ob, ref[real], rows=real)
    assert (host_bits(ob)[gap] == 0).all()
    assert np.abs(ls.cpu().numpy().T[real] - ref_lse[real]).max() < 5e-3


def test_padding_content_changes_nothing(pvc):
    w = make_workload("sft", scale="small")
    cu, cp = _layout(w.lengths, 64)
    Ts, H, d = int(cp[-1]), w.heads, w.head_dim
    q, k, v = (_bits((Ts, H, d), s) for s in (4, 5, 6))
    _, _, ob1, _, _ = _fwd(pvc, q, k, v, cu, cp)
    gap = np.setdiff1d(np.arange(Ts), A.storage_rows(cu, cp))
    for x, seed in ((q, 7), (k, 8), (v, 9)):
        x[gap] = _bits((gap.size, H, d), seed, 50.0)
    _, _, ob2, _, _ = _fwd(pvc, q, k, v, cu, cp)
    assert (host_bits(ob1) == host_bits(ob2)).all()


@pytest.mark.parametrize("causal", [True, False])
def test_backward(pvc, causal):
    w = make_workload("sft", scale="small")
    cu, cp = _layout(w.lengths, 64)
    Ts, H, d = int(cp[-1]), w.heads, w.head_dim
    say(f"  padded bwd causal={causal}: T={w.total_tokens} storage={Ts}")
    q, k, v, g = (_bits((Ts, H, d), s) for s in (11, 12, 13, 14))
    plan, (qd, kd, vd), ob, _, ls = _fwd(pvc, q, k, v, cu, cp, causal)
    gd = dev_bf16(g)
    g32 = pvc.varlen_attn_bwd(qd, kd, vd, ob, gd, ls, plan, causal, grad_dtype=torch.float32)
    g16 = pvc.varlen_attn_bwd(qd, kd, vd, ob, gd, ls, plan, causal)
    torch.cuda.synchronize()
    refs = A.attention_bwd_padded(q, k, v, g, cu, cp, causal, threads=16)
    real = A.storage_rows(cu, cp)
    gap = np.setdiff1d(np.arange(Ts), real)
    bc = grad_error_bounds(q[real], k[real], v[real], g[real], cu, causal)
    bounds = []
    for b in bc:
        full = np.zeros((Ts, H, d))
        full[real] = b
        bounds.append(full)
    grad_check(g32, g16, refs, bounds, rows=real)
    for t in g32:
        assert (t.cpu().numpy()[gap] == 0).all()


def test_rope_with_padded_cu(pvc):
    w = make_workload("sft", scale="small")
    cu, cp = _layout(w.lengths, 64)
    Ts, H, d = int(cp[-1]), w.heads, w.head_dim
    x = _bits((Ts, H, d), 21)
    xd = dev_bf16(x)
    pvc.rope_thd_apply(xd, None, dev_i32(cp), w.rope_base)
    torch.cuda.synchronize()
    real = A.storage_rows(cu, cp)
    ref = R.rope_apply(x[real], cu, w.rope_base)         # compact buffer, positions from each segment start
    assert (host_bits(xd)[real] == ref).all()


def test_short_slot_is_refused(pvc):
    lengths = [30, 20, 14]
    cu, cp = _layout(lengths, 32)
    cp_bad = cp.copy()
    cp_bad[1] = 16                                         # slot 0 shorter than its 30 tokens
    Ts, H, d = int(cp[-1]), 2, 64
    q, k, v = (dev_bf16(_bits((Ts, H, d), s)) for s in (1, 2, 3))
    plan = pvc.attn_plan(dev_i32(cu), Ts, 30, True, cu_seqlens_padded=dev_i32(cp_bad))
    out = torch.full((Ts, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    pvc.varlen_attn_fwd(q, k, v, plan=plan, out=out)
    torch.cuda.synchronize()
    assert int(plan.dev_error.item()) & 512
    assert (out.float() == 7.0).all()
