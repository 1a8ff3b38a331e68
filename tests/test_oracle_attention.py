"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against: the pages' zero-score example (10 isolated,
3.25 whole-pack), PyTorch's CPU scaled_dot_product_attention on special cases
(bool mask with True = attend, and is_causal for a single segment), closed
forms (single-key rows, constant V), invariants (packed == unpacked, changing
segment A leaves B and C untouched), and brute force on tiny inputs.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import pack as P
from oracle.rope import bf16_bits_to_f64, f64_to_bf16_bits
from workloads import make_workload, qkv_bits


def _bits(x):
    return f64_to_bf16_bits(np.asarray(x, np.float64))


def _rand(T, H, d, seed):
    rng = np.random.default_rng(seed)
    return [_bits(rng.standard_normal((T, H, d))) for _ in range(3)]


def _sdpa(q, k, v, mask=None, is_causal=False):
    Q, K, V = (torch.from_numpy(bf16_bits_to_f64(x)).permute(1, 0, 2) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=m, is_causal=is_causal)
    return o.permute(1, 0, 2).numpy()


def test_zero_score_example(golden):
    case = golden("attention_examples.json")["zero_score"]
    T, H, d = 9, 2, 64
    q = _bits(np.zeros((T, H, d)))
    k = _bits(np.random.default_rng(0).standard_normal((T, H, d)))
    v = np.zeros((T, H, d))
    v[0:3] = case["v_A"]
    v[3] = case["v_b0"]
    v = _bits(v)
    cu = P.pack_build(case["lengths"])["cu_seqlens"]
    o_iso, _ = A.attention(q, k, v, cu)
    o_pack, _ = A.attention(q, k, v, [0, T])
    assert (o_iso[3] == case["expected_b0_isolated"]).all()
    assert (o_pack[3] == case["expected_b0_whole_pack"]).all()
    ob, _ = A.attention_brute(q, k, v, cu)
    assert (ob[3] == case["expected_b0_isolated"]).all()


@pytest.mark.parametrize("lengths,causal", [([3, 2, 4], True), ([1, 5, 2, 7, 1], True),
                                            ([3, 2, 4], False), ([6, 10], False), ([16], True)])
def test_brute_mask_vs_torch_sdpa_bool_mask(lengths, causal):
    """Explicit mask, True = attend (the PyTorch SDPA boolean convention)."""
    T = sum(lengths)
    q, k, v = _rand(T, 3, 32, T)
    cu = P.pack_build(lengths)["cu_seqlens"]
    allow = A.allow_matrix(cu, causal)
    ref = _sdpa(q, k, v, mask=allow)
    ob, _ = A.attention_brute(q, k, v, cu, causal)
    oc, _ = A.attention(q, k, v, cu, causal)
    np.testing.assert_allclose(ob, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oc, ref, rtol=0, atol=1e-12)


def test_allow_matrix_shape_is_block_diagonal_lower():
    allow = A.allow_matrix([0, 3, 5, 9])
    # A3 (row 2) sees A1..A3; B1 (row 3) sees only itself; C sees nothing of A or B
    assert allow[2, :3].all() and not allow[2, 3:].any()
    assert allow[3].tolist() == [False] * 3 + [True] + [False] * 5
    assert not allow[5:, :5].any()
    assert allow.sum() == 19                                # [charlestar] two ledgers: 19 pairs


def test_single_segment_is_textbook_causal():
    T = 40
    q, k, v = _rand(T, 2, 64, 3)
    ref = _sdpa(q, k, v, is_causal=True)
    oc, _ = A.attention(q, k, v, [0, T])
    np.testing.assert_allclose(oc, ref, rtol=0, atol=1e-12)


def test_lse_matches_logsumexp():
    lengths = [5, 1, 9]
    T = sum(lengths)
    q, k, v = _rand(T, 2, 64, 11)
    cu = P.pack_build(lengths)["cu_seqlens"]
    _, lse = A.attention(q, k, v, cu)
    Q, K = bf16_bits_to_f64(q), bf16_bits_to_f64(k)
    allow = A.allow_matrix(cu)
    for h in range(2):
        S = torch.from_numpy(Q[:, h] @ K[:, h].T / 8.0)
        S[~torch.from_numpy(allow)] = -torch.inf
        np.testing.assert_allclose(lse[:, h], torch.logsumexp(S, dim=1).numpy(), rtol=0, atol=1e-12)


def test_single_key_rows_and_constant_v():
    w = make_workload("short", scale="small")
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    starts = cu[:-1].astype(np.int64)
    o, _ = A.attention_rows(q, k, v, cu, starts)
    assert (o == bf16_bits_to_f64(v[starts])).all()         # softmax over one key is 1
    vc = _bits(np.full(v.shape, 1.375))
    rows = np.arange(0, w.total_tokens, 37, dtype=np.int64)
    oc, _ = A.attention_rows(q, k, vc, cu, rows)
    np.testing.assert_allclose(oc, 1.375, rtol=1e-15, atol=0)


def test_packed_equals_unpacked_bitwise():
    w = make_workload("sft", scale="small", heads=1)
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    o, lse = A.attention(q, k, v, cu, threads=4)
    ou, lseu = A.attention_unpacked(q, k, v, cu, threads=4)
    assert (o == ou).all() and (lse == lseu).all()


def test_changing_a_leaves_others_untouched():
    lengths = [7, 5, 9]
    T = sum(lengths)
    q, k, v = _rand(T, 2, 64, 5)
    cu = P.pack_build(lengths)["cu_seqlens"]
    o1, _ = A.attention(q, k, v, cu)
    q2, k2, v2 = (x.copy() for x in (q, k, v))
    rng = np.random.default_rng(9)
    for x in (q2, k2, v2):
        x[:7] = _bits(rng.standard_normal(x[:7].shape) * 3)
    o2, _ = A.attention(q2, k2, v2, cu)
    assert (o1[7:] == o2[7:]).all()
    assert (o1[:7] != o2[:7]).any()
    # whole-pack causal attention would leak A into B and C
    o3, _ = A.attention(q, k, v, [0, T])
    o4, _ = A.attention(q2, k2, v2, [0, T])
    assert (o3[7:] != o4[7:]).any()


def test_threads_do_not_change_results():
    w = make_workload("pretrain", scale="small", heads=1)
    q, k, v = w.qkv()
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    rows = np.arange(0, w.total_tokens, 13, dtype=np.int64)
    a, la = A.attention_rows(q, k, v, cu, rows, threads=1)
    b, lb = A.attention_rows(q, k, v, cu, rows, threads=6)
    assert (a == b).all() and (la == lb).all()
