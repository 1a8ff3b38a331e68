"""GPU parity for rope_thd_apply: bit-exact against the fp64 oracle (both round
the rotation, evaluated in double, once to bf16); an element whose exact value
sits within the double evaluation error of a bf16 tie may differ by one ulp."""

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


def _near_tie(x_bits: np.ndarray, positions, base: float, interleaved: bool = False) -> np.ndarray:
    """Elements whose exact rotated value lies so close to a bf16 rounding
    midpoint that two correct double evaluations may round to different
    neighbours: distance to the midpoint below the double evaluation's error
    bound, 8 * 2^-53 * (|x_j| + |x_{j+d/2}|), measured in bf16 ulps."""
    d = x_bits.shape[-1]
    x = R.bf16_bits_to_f64(x_bits)
    if interleaved:
        y = R.rotate_interleaved_f64(x, R.rope_angles(positions, d, base))
        mag = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
    else:
        y = R.rotate_f64(x, R.rope_angles(positions, d, base))
        mag = np.abs(x[..., : d // 2]) + np.abs(x[..., d // 2:])
        mag = np.concatenate([mag, mag], axis=-1)
    ay = np.abs(y)
    e = np.floor(np.log2(np.where(ay > 0, ay, 1.0)))
    ulp = np.exp2(e - 7)
    frac = ay / ulp - np.floor(ay / ulp)           # position between bf16 neighbours
    tol = 8 * 2.0 ** -53 * mag / ulp
    return np.abs(frac - 0.5) <= tol


def _check(got_bits, ref_bits, what, x_bits=None, positions=None, base=10000.0, interleaved=False):
    """Bit-exact except near-tie elements (at most one ulp there)."""
    d = _ulp_diff(got_bits, ref_bits)
    near = (_near_tie(x_bits, positions, base, interleaved) if x_bits is not None
            else np.zeros(d.shape, bool))
    say(f"    {what}: {int((d > 0).sum())} of {d.size} elements differ (max {int(d.max())} ulp); "
        f"near-tie elements {int(near.sum())}")
    assert d.max() <= 1, what
    assert (d[~near] == 0).all(), what


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
    pos = P.positions_from_cu(cu)
    _check(gq, R.rope_apply(q, cu, w.rope_base), "q", q, pos, w.rope_base)
    _check(gk, R.rope_apply(k, cu, w.rope_base), "k", k, pos, w.rope_base)
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
    pos = P.positions_from_cu(cu)[rows]
    _check(gq[rows], R.rope_apply(q, cu, w.rope_base, rows=rows), "q sampled", q[rows], pos, w.rope_base)
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
    _check(host_bits(qd), R.rope_apply(q, cu, 500.0), f"d={d}", q, P.positions_from_cu(cu), 500.0)


def test_malformed_cu_sets_bits_and_copies(pvc):
    q = np.random.default_rng(1).integers(0x3000, 0x4000, (9, 2, 64)).astype(np.uint16)
    qd = dev_bf16(q)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pvc.rope_thd_apply(qd, None, dev_i32([0, 3, 5, 7]), dev_error=err)   # tokens 7, 8 in no segment
    torch.cuda.synchronize()
    assert int(err.item()) & P.ERR_TOTAL
    assert (host_bits(qd)[7:] == q[7:]).all()


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_interleaved_small_workloads_all_tokens(pvc, name):
    w = make_workload(name, scale="small")
    say(f"  rope interleaved small {name}: T={w.total_tokens} H={w.heads} d={w.head_dim}")
    q, k = qkv_bits(w, "q"), qkv_bits(w, "k")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd, kd = dev_bf16(q), dev_bf16(k)
    pvc.rope_thd_apply(qd, kd, dev_i32(cu), w.rope_base, interleaved=True)
    torch.cuda.synchronize()
    pos = P.positions_from_cu(cu)
    for got, x, what in ((host_bits(qd), q, "q"), (host_bits(kd), k, "k")):
        _check(got, R.rope_apply(x, cu, w.rope_base, interleaved=True), what, x, pos, w.rope_base, True)
        assert (got[cu[:-1]] == x[cu[:-1]]).all()


@pytest.mark.parametrize("d", [8, 48, 96, 128])
def test_interleaved_head_dims(pvc, d):
    """d = 8: one pair per thread; d % 16 == 0: the vectorized four-pair path."""
    lengths = [5, 17, 300, 1]
    T = sum(lengths)
    from workloads import f32_to_bf16_bits
    q = f32_to_bf16_bits(np.random.default_rng(d + 1).standard_normal((T, 3, d), dtype=np.float32))
    cu = P.pack_build(lengths)["cu_seqlens"]
    qd = dev_bf16(q)
    pvc.rope_thd_apply(qd, None, dev_i32(cu), 500.0, interleaved=True)
    torch.cuda.synchronize()
    _check(host_bits(qd), R.rope_apply(q, cu, 500.0, interleaved=True), f"interleaved d={d}", q,
           P.positions_from_cu(cu), 500.0, True)


def test_interleaved_full_size_sampled_tokens(pvc):
    w = make_workload("sft")
    q = qkv_bits(w, "q")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    qd = dev_bf16(q)
    pvc.rope_thd_apply(qd, None, dev_i32(cu), w.rope_base, interleaved=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, np.random.default_rng(2).integers(0, w.total_tokens, 3000)]))
    pos = P.positions_from_cu(cu)[rows]
    _check(host_bits(qd)[rows], R.rope_apply(q, cu, w.rope_base, rows=rows, interleaved=True),
           "interleaved q sampled", q[rows], pos, w.rope_base, True)
