"""GPU parity for fp16 inputs ([charlestar] "varlen interface": q, k, v in fp16
or bf16): the attention forward (self and prefill plans), its backward, RoPE
and the packed cross-entropy, each against the fp64 oracle on the fp16 values.

Attention: the fp32 output within 1e-2 max-abs of the oracle and the fp16
output equal to the nearest-even fp16 rounding of the fp32 output.  Backward:
fp32 gradients within the first-order bounds of the bf16 tests with fp16's
unit roundoff and absolute floor, fp16 gradients the RNE of the fp32 ones.  RoPE:
bit-exact fp16 results (one ulp allowed only where the exact value lies within
the double evaluation's error of an fp16 rounding midpoint).  CE: row losses
within the bound of the bf16 tests, counts exact, fp16 gradient the RNE of the
fp32 gradient.
"""

import numpy as np
import pytest
import torch

from gpu_util import ATOL, dev_i32, grad_check, grad_error_bounds, say
from oracle import attention as A
from oracle import loss as L
from oracle import pack as P
from oracle import rope as R
from test_gpu_5_ce import row_bound
from workloads import make_prefill, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _f16(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float16)


def _dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16)).cuda()


def _check_f16(of, oh, ref, rows=None):
    f32 = of.cpu().numpy().astype(np.float64)
    h = oh.cpu().numpy()
    if rows is not None:
        f32, h = f32[rows], h[rows]
    err = np.abs(f32 - ref).max()
    rne = f32.astype(np.float32).astype(np.float16)
    mism = int((rne.view(np.uint16) != h.view(np.uint16)).sum())
    raw = np.abs(h.astype(np.float64) - ref).max()
    say(f"    fp16 parity: max abs fp32 {err:.3e}, fp16 vs RNE mismatches {mism}, raw fp16 {raw:.3e}")
    assert err <= ATOL and mism == 0


@pytest.mark.parametrize("name", ["sft", "short", "longctx"])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_fp16_small(pvc, name, causal):
    w = make_workload(name, scale="small")
    T, H, d = w.total_tokens, w.heads, w.head_dim
    say(f"  fp16 attn {name} causal={causal}: T={T} H={H} d={d}")
    q, k, v = (_f16((T, H, d), s) for s in (1, 2, 3))
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    plan = pvc.attn_plan(dev_i32(cu), T, int(w.lengths.max()), causal)
    oh = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal)
    of, ls = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert oh.dtype == torch.float16 and int(plan.dev_error.item()) == 0
    ref, ref_lse = A.attention_qk(q, k, v, cu, cu, causal)
    _check_f16(of, oh, ref)
    assert np.abs(ls.cpu().numpy().T - ref_lse).max() < 5e-3


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_fp16(pvc, causal, d):
    w = make_workload("sft", scale="small")
    T, H = w.total_tokens, w.heads
    say(f"  fp16 bwd causal={causal} d={d}: T={T} H={H}")
    q, k, v, g = (_f16((T, H, d), s) for s in (11, 12, 13, 14))
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd, vd, gd = _dev(q), _dev(k), _dev(v), _dev(g)
    plan = pvc.attn_plan(dev_i32(cu), T, int(w.lengths.max()), causal)
    out, lse = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, return_lse=True)
    g32 = pvc.varlen_attn_bwd(qd, kd, vd, out, gd, lse, plan, causal, grad_dtype=torch.float32)
    g16 = pvc.varlen_attn_bwd(qd, kd, vd, out, gd, lse, plan, causal)
    torch.cuda.synchronize()
    assert all(t.dtype == torch.float16 for t in g16) and int(plan.dev_error.item()) == 0
    refs = A.attention_bwd(q, k, v, g, cu, causal, threads=16)
    grad_check(g32, g16, refs, grad_error_bounds(q, k, v, g, cu, causal, f16=True))


def test_backward_fp16_refuses_mixed_types(pvc):
    w = make_workload("tiny")
    T, H, d = w.total_tokens, w.heads, w.head_dim
    q = _dev(_f16((T, H, d), 1))
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    plan = pvc.attn_plan(dev_i32(cu), T, int(w.lengths.max()), True)
    out, lse = pvc.varlen_attn_fwd(q, q, q, plan=plan, return_lse=True)
    with pytest.raises(TypeError):
        pvc.varlen_attn_bwd(q, q, q, out.to(torch.bfloat16), q, lse, plan)
    with pytest.raises(TypeError):
        pvc.varlen_attn_bwd(q, q, q, out, q, lse, plan, grad_dtype=torch.bfloat16)


@pytest.mark.parametrize("heads,kv_heads", [(4, 2), (8, 2)])
def test_prefill_fp16(pvc, heads, kv_heads):
    """The small prefill in fp16, with 2 query heads per key / value head
    and with 4 (four query heads per workgroup)."""
    pw = make_prefill(scale="small")
    pw.heads, pw.kv_heads = heads, kv_heads
    q = _f16((pw.total_q, pw.heads, pw.head_dim), 4)
    k, v = _f16((pw.total_k, pw.kv_heads, pw.head_dim), 5), _f16((pw.total_k, pw.kv_heads, pw.head_dim), 6)
    cu_q = np.concatenate([[0], np.cumsum(pw.lq)])
    cu_k = np.concatenate([[0], np.cumsum(pw.lk)])
    say(f"  fp16 prefill Tq={pw.total_q} Tk={pw.total_k}")
    plan = pvc.attn_plan_qk(dev_i32(cu_q), dev_i32(cu_k), pw.total_q, pw.total_k, int(pw.lq.max()),
                            int(pw.lk.max()), True)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    oh = pvc.varlen_attn_fwd_qk(qd, kd, vd, plan=plan)
    of = pvc.varlen_attn_fwd_qk(qd, kd, vd, plan=plan, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = A.attention_qk(q, k, v, cu_q, cu_k, True)
    _check_f16(of, oh, ref)


def _near_tie_f16(x16, positions, base, interleaved):
    d = x16.shape[-1]
    x = x16.astype(np.float64)
    theta = R.rope_angles(positions, d, base)
    if interleaved:
        y = R.rotate_interleaved_f64(x, theta)
        mag = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
    else:
        y = R.rotate_f64(x, theta)
        mag = np.abs(x[..., : d // 2]) + np.abs(x[..., d // 2:])
        mag = np.concatenate([mag, mag], axis=-1)
    ay = np.abs(y)
    e = np.maximum(np.floor(np.log2(np.where(ay > 0, ay, 1.0))), -14)
    ulp = np.exp2(e - 10)
    frac = ay / ulp - np.floor(ay / ulp)
    return np.abs(frac - 0.5) <= 8 * 2.0 ** -53 * mag / ulp


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("d", [128, 48, 10])
def test_rope_fp16(pvc, interleaved, d):
    lengths = [5, 17, 300, 1, 90]
    T = sum(lengths)
    x = _f16((T, 3, d), d, 3.0)
    cu = P.pack_build(lengths)["cu_seqlens"]
    xd = _dev(x)
    pvc.rope_thd_apply(xd, None, dev_i32(cu), 500.0, interleaved=interleaved)
    torch.cuda.synchronize()
    got = xd.cpu().numpy().view(np.uint16)
    ref = R.rope_apply(x.view(np.uint16), cu, 500.0, interleaved=interleaved, f16=True)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    near = _near_tie_f16(x, P.positions_from_cu(cu), 500.0, interleaved)
    say(f"    fp16 rope d={d} interleaved={interleaved}: {int((diff > 0).sum())} differ, near-tie {int(near.sum())}")
    assert (diff[~near] == 0).all() and diff.max() <= 1
    assert (got[cu[:-1]] == x.view(np.uint16)[cu[:-1]]).all()


def test_cross_entropy_fp16_logits_and_gradient(pvc):
    w = make_workload("sft", scale="small")
    V, T = 32000, w.total_tokens
    z = _f16((T, V), 7, 2.0)
    meta = P.pack_build(w.lengths, w.tokens(), w.is_pad)
    lab = meta["shifted_labels"]
    zd = _dev(z)
    out = pvc.packed_ce_loss(zd, dev_i32(lab), dev_i32(meta["cu_seqlens"]), row_loss=True, segments=True,
                             grad="new", grad_dtype=torch.float32, grad_scale=0.5)
    o16 = pvc.packed_ce_loss(zd, dev_i32(lab), grad="new", grad_scale=0.5)
    torch.cuda.synchronize()
    ref = L.packed_loss(z, lab, meta["cu_seqlens"])
    rl = out["row_loss"].cpu().numpy().astype(np.float64)
    bound = row_bound(z.astype(np.float64), ref["row_loss"])
    err = np.abs(rl - ref["row_loss"])
    say(f"  fp16 CE: max row err {err.max():.3e}, max err / bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    assert int(out["target_count"].item()) == ref["target_count"]
    assert (out["seg_count"].cpu().numpy() == ref["seg_count"]).all()
    g32 = out["grad"].cpu().numpy()
    assert o16["grad"].dtype == torch.float16
    assert (g32.astype(np.float16).view(np.uint16) == o16["grad"].cpu().numpy().view(np.uint16)).all()
    rows = np.arange(0, T, 97)
    gref = L.loss_grad(z[rows], lab[rows], 0.5)
    assert np.abs(g32[rows] - gref).max() < 1e-6
