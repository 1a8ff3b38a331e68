"""Pins of the prefill attention oracle (separate query / key boundaries,
grouped key-value heads; CPU only)."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.rope import bf16_bits_to_f64
from workloads import f32_to_bf16_bits


def _bits(shape, seed):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


@pytest.mark.parametrize("causal", [True, False])
def test_square_boundaries_and_no_grouping_equal_the_self_attention_oracle(causal):
    cu = np.array([0, 5, 6, 19, 40])
    q, k, v = (_bits((40, 2, 16), s) for s in (1, 2, 3))
    a, la = A.attention_qk(q, k, v, cu, cu, causal)
    b, lb = A.attention(q, k, v, cu, causal)
    assert np.abs(a - b).max() < 1e-12 and np.abs(la - lb).max() < 1e-12


def test_bottom_right_alignment_against_sdpa_with_an_explicit_mask():
    """Each request through PyTorch SDPA with the bool mask j <= i + Lk - Lq."""
    cu_q = np.array([0, 3, 4, 10])
    cu_k = np.array([0, 8, 12, 18])          # Lk - Lq = 5, 3, 0
    q = _bits((10, 4, 16), 4)
    k, v = _bits((18, 2, 16), 5), _bits((18, 2, 16), 6)
    out, _ = A.attention_qk(q, k, v, cu_q, cu_k, True)
    Q, K, V = (torch.from_numpy(bf16_bits_to_f64(x)) for x in (q, k, v))
    for r in range(3):
        qs, qe, ks, ke = cu_q[r], cu_q[r + 1], cu_k[r], cu_k[r + 1]
        Lq, Lk = qe - qs, ke - ks
        mask = torch.arange(Lk)[None, :] <= torch.arange(Lq)[:, None] + (Lk - Lq)
        for h in range(4):
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[qs:qe, h][None], K[ks:ke, h // 2][None], V[ks:ke, h // 2][None], attn_mask=mask[None])[0]
            assert np.abs(out[qs:qe, h] - ref.numpy()).max() < 1e-12
    # the last query of every request sees all of its keys
    allk, _ = A.attention_qk(q, k, v, cu_q, cu_k, False)
    last = cu_q[1:] - 1
    assert np.abs(out[last] - allk[last]).max() < 1e-12


def test_grouped_heads_equal_repeated_kv_heads():
    cu_q, cu_k = np.array([0, 7, 9]), np.array([0, 12, 20])
    q = _bits((9, 6, 16), 7)
    k, v = _bits((20, 2, 16), 8), _bits((20, 2, 16), 9)
    a, _ = A.attention_qk(q, k, v, cu_q, cu_k, True)
    b, _ = A.attention_qk(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu_q, cu_k, True)
    assert np.array_equal(a, b)


def test_queries_without_keys_and_single_query_decode():
    cu_q, cu_k = np.array([0, 5, 6]), np.array([0, 3, 9])      # request 0: 5 queries over 3 keys
    q = _bits((6, 1, 8), 10)
    k, v = _bits((9, 1, 8), 11), _bits((9, 1, 8), 12)
    out, lse = A.attention_qk(q, k, v, cu_q, cu_k, True)
    assert (out[:2] == 0).all() and np.isneginf(lse[:2]).all()   # a + 3 - 5 + 1 <= 0 for a < 2
    assert np.isfinite(lse[2:]).all()
    # request 1 is one query over 6 keys (decode): it attends to all of them
    V = bf16_bits_to_f64(v)[3:9, 0]
    sc = bf16_bits_to_f64(k)[3:9, 0] @ bf16_bits_to_f64(q)[5, 0] / np.sqrt(8)
    p = np.exp(sc - sc.max())
    assert np.abs(out[5, 0] - p @ V / p.sum()).max() < 1e-12
