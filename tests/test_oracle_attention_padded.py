"""Pins of the padded-storage attention oracle (CPU only): the C loop on the
compacted buffer, scattered through the offset map, against an explicit
storage x storage mask in numpy; gradients against PyTorch float64 autograd of
that masked form; padding rows are 0 / -inf / zero gradients."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.rope import bf16_bits_to_f64
from workloads import f32_to_bf16_bits

CASES = [
    ([3, 2, 4], [0, 4, 8, 12]),          # every slot padded to 4
    ([5, 1, 7], [0, 5, 8, 16]),          # first slot exact, others padded
    ([1, 1], [0, 2, 4]),
]


def _qkv(T, H=2, d=8, seed=0):
    """bf16 bit patterns (what the C loop takes) of N(0,1) draws."""
    rng = np.random.default_rng(seed)
    return tuple(f32_to_bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32)) for _ in range(4))


@pytest.mark.parametrize("lengths,cp", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_padded_matches_explicit_storage_mask(lengths, cp, causal):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Ts = cp[-1]
    q, k, v, _ = _qkv(Ts)
    o, ls = A.attention_padded(q, k, v, cu, cp, causal)
    ob, lb = A.attention_brute_masked(q, k, v, A.allow_matrix_padded(cu, cp, Ts, causal))
    assert np.abs(o - ob).max() < 1e-12
    fin = np.isfinite(lb)
    assert (np.isfinite(ls) == fin).all() and np.abs(ls[fin] - lb[fin]).max() < 1e-12
    real = A.storage_rows(cu, cp)
    gap = np.setdiff1d(np.arange(Ts), real)
    assert (o[gap] == 0).all() and np.isneginf(ls[gap]).all()


def test_padding_content_does_not_matter():
    cu, cp = np.array([0, 3, 5, 9]), np.array([0, 4, 8, 12])
    q, k, v, _ = _qkv(12, seed=3)
    gap = np.setdiff1d(np.arange(12), A.storage_rows(cu, cp))
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[gap] = 0x4480                          # bf16 1024
    a, _ = A.attention_padded(q, k, v, cu, cp)
    b, _ = A.attention_padded(q2, k2, v2, cu, cp)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("lengths,cp", CASES)
def test_padded_gradients_match_autograd_of_the_masked_form(lengths, cp):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Ts = cp[-1]
    q, k, v, g = _qkv(Ts, seed=5)
    dq, dk, dv = A.attention_bwd_padded(q, k, v, g, cu, cp, True)
    allow = torch.from_numpy(A.allow_matrix_padded(cu, cp, Ts, True))
    has = allow.any(dim=1)
    Q, K, V = (torch.from_numpy(bf16_bits_to_f64(x)).requires_grad_() for x in (q, k, v))
    outs = []
    for h in range(q.shape[1]):
        S = Q[:, h] @ K[:, h].T / np.sqrt(q.shape[2])
        S = S.masked_fill(~allow, float("-inf"))[has]
        outs.append(torch.softmax(S, dim=1) @ V[:, h])
    G = bf16_bits_to_f64(g)
    loss = sum((o * torch.from_numpy(G[has.numpy(), h])).sum() for h, o in enumerate(outs))
    loss.backward()
    for a, b in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12
