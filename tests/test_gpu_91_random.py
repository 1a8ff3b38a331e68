"""Seeded random packs through the GPU path, against the fp64 oracle.

Each case draws a segment count, a length for every segment from a mix of
very short, mid and long samples, a head count (some multiples of 8, which
take the head-interleaved item order), a head dim and the causal flag.
Checks:
  - forward: every element with the three-part check of the other tests and
    the LSE within 5e-3;
  - backward: every gradient element within its first-order bound, 16-bit
    gradients the RNE of the fp32 ones;
  - pack_build on the same lengths: bit-exact.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev_bf16, dev_i32, grad_check, grad_error_bounds, say, three_part_check
from oracle import attention as A
from oracle import pack as P
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _case(seed):
    rng = np.random.default_rng([91, seed])
    n = int(rng.integers(1, 30))
    kind = rng.integers(0, 3, n)                  # 0: 1-8 tokens, 1: 9-200, 2: 201-700
    lo = np.array([1, 9, 201])[kind]
    hi = np.array([9, 201, 701])[kind]
    lengths = rng.integers(lo, hi)
    H = int(rng.choice([2, 3, 8, 16]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    return rng, lengths, H, d, causal


def _bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@pytest.mark.parametrize("seed", range(8))
def test_random_pack_forward_backward(pvc, seed):
    rng, lengths, H, d, causal = _case(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    say(f"  random case {seed}: nseg={lengths.size} T={T} max={int(lengths.max())} H={H} d={d} causal={causal}")
    q, k, v, g = (_bits(rng, (T, H, d)) for _ in range(4))
    qd, kd, vd, gd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(g)

    meta = pvc.pack_build(dev_i32(lengths), total_tokens=T)
    plan = pvc.attn_plan(meta["cu_seqlens"], T, int(lengths.max()), causal)
    ob, lse = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, return_lse=True)
    of = pvc.varlen_attn_fwd(qd, kd, vd, plan=plan, causal=causal, out_dtype=torch.float32)
    g32 = pvc.varlen_attn_bwd(qd, kd, vd, ob, gd, lse, plan, causal, grad_dtype=torch.float32)
    g16 = pvc.varlen_attn_bwd(qd, kd, vd, ob, gd, lse, plan, causal)
    torch.cuda.synchronize()
    assert int(meta["dev_error"].item()) == 0 and int(plan.dev_error.item()) == 0

    ref = P.pack_build(lengths)
    assert (meta["cu_seqlens"].cpu().numpy() == ref["cu_seqlens"]).all()
    assert (meta["position_ids"].cpu().numpy() == ref["position_ids"]).all()

    out_ref, lse_ref = A.attention(q, k, v, cu, causal, threads=16)
    three_part_check(of, ob, out_ref)
    assert np.abs(lse.cpu().numpy().T - lse_ref).max() < 5e-3

    refs = A.attention_bwd(q, k, v, g, cu, causal, threads=16)
    grad_check(g32, g16, refs, grad_error_bounds(q, k, v, g, cu, causal))
