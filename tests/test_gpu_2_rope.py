"""GPU parity for rope_thd_apply: within one bf16 ulp of the fp64 oracle, and
bit-exact where the pages fix the result (position 0, per-segment reset)."""

import numpy as np
import pytest
import torch

from gpu_util import dev_bf16, dev_i32, host_bits, say
from oracle import pack as P
from oracle import rope as R
from workloads import CONFIG_NAMES, make_workload, qkv_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two bf16 bit arrays (same-sign ordering)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a) - key(b))


def _check(got_bits, ref_bits, what):
    d = _ulp_diff(got_bits, ref_bits)
    n1 = int((d == 1).sum())
    say(f"    {what}: max ulp {int(d.max())}, elements off by 1 ulp: {n1} of {d.size}")
    assert d.max() <= 1, what


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_small_workloads_all_tokens(pvc, name):
    w = make_workload(name, scale="small")
    say(f"  rope small {name}: T={w.total_tokens} H={w.heads} d={w.head_dim}")
    q, k = qkv_bits(w, "q"), qkv_bits(w, "k")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd = dev_bf16(q), dev_bf16(k)
    pvc.rope_thd_apply(qd, kd, dev_i32(cu), w.rope_base)
    torch.cuda.synchronize()
    gq, gk = host_bits(qd), host_bits(kd)
    _check(gq, R.rope_apply(q, cu, w.rope_base), "q")
    _check(gk, R.rope_apply(k, cu, w.rope_base), "k")
    starts = cu[:-1]
    assert (gq[starts] == q[starts]).all() and (gk[starts] == k[starts]).all()   # p = 0 identity


@pytest.mark.parametrize("name", ["sft", "pretrain", "longctx", "short"])
def test_full_size_sampled_tokens(pvc, name):
    w = make_workload(name)
    say(f"  rope full {name}: T={w.total_tokens} H={w.heads} d={w.head_dim}")
    q = qkv_bits(w, "q")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd = dev_bf16(q)
    kd = qd.clone()
    pvc.rope_thd_apply(qd, kd, dev_i32(cu), w.rope_base)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, rng.integers(0, w.total_tokens, 3000)]))
    gq = host_bits(qd)
    _check(gq[rows], R.rope_apply(q, cu, w.rope_base, rows=rows), "q sampled")
    assert (host_bits(kd) == gq).all()          # same input, same kernel: identical
    assert (gq[cu[:-1]] == q[cu[:-1]]).all()


def test_out_of_place_and_q_only(pvc):
    w = make_workload("sft", scale="small")
    q, k = qkv_bits(w, "q"), qkv_bits(w, "k")
    cu = dev_i32(P.pack_build(w.lengths)["cu_seqlens"])
    qd, kd = dev_bf16(q), dev_bf16(k)
    qo, ko = torch.empty_like(qd), torch.empty_like(kd)
    pvc.rope_thd_apply(qd, kd, cu, q_out=qo, k_out=ko)
    q2 = dev_bf16(q)
    pvc.rope_thd_apply(q2, None, cu)
    torch.cuda.synchronize()
    assert (host_bits(qd) == q).all() and (host_bits(kd) == k).all()   # inputs untouched
    assert (host_bits(qo) == host_bits(q2)).all()


def test_segment_reset_matches_standalone(pvc):
    """RoPE of a segment inside the pack == RoPE of that segment alone, bit for bit."""
    w = make_workload("longctx", scale="small")
    q = qkv_bits(w, "q")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    packed = dev_bf16(q)
    pvc.rope_thd_apply(packed, None, dev_i32(cu))
    gp = host_bits(packed)
    for r in range(0, w.nseg, 3):
        s, e = int(cu[r]), int(cu[r + 1])
        alone = dev_bf16(q[s:e])
        pvc.rope_thd_apply(alone, None, dev_i32([0, e - s]))
        assert (host_bits(alone) == gp[s:e]).all()


@pytest.mark.parametrize("d", [8, 48, 96])
def test_other_head_dims(pvc, d):
    lengths = [5, 17, 300, 1]
    T = sum(lengths)
    rng = np.random.default_rng(d)
    from workloads import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((T, 3, d), dtype=np.float32))
    cu = P.pack_build(lengths)["cu_seqlens"]
    qd = dev_bf16(q)
    pvc.rope_thd_apply(qd, None, dev_i32(cu), 500.0)
    torch.cuda.synchronize()
    _check(host_bits(qd), R.rope_apply(q, cu, 500.0), f"d={d}")


def test_malformed_cu_sets_bits_and_copies(pvc):
    q = np.random.default_rng(1).integers(0x3000, 0x4000, (9, 2, 64)).astype(np.uint16)
    qd = dev_bf16(q)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pvc.rope_thd_apply(qd, None, dev_i32([0, 3, 5, 7]), dev_error=err)   # tokens 7, 8 in no segment
    torch.cuda.synchronize()
    assert int(err.item()) & P.ERR_TOTAL
    assert (host_bits(qd)[7:] == q[7:]).all()
