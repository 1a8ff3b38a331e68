"""Pins for the fp64 attention-gradient oracle (CPU only).

The gradient oracle (oracle.attention.attention_bwd, the C loop
oracle_attn_bwd_segment) is pinned to things other than itself:
  - PyTorch autograd in float64 through an explicit additive-mask attention
    (the definition of [charlestar] "EOS is content", differentiated by the
    library);
  - central finite differences of the forward oracle (attention_brute, itself
    pinned to scaled_dot_product_attention in test_oracle_attention.py);
  - closed forms: a query that sees one key has dQ = 0; a one-token segment has
    dK = 0 and dV = dO; with q = 0 every visible key has the same weight, so
    dK = 0 and dV_j = sum over i >= j of dO_i / (i - start + 1);
  - packing: a segment's gradients equal those of the segment alone, bit for
    bit ([charlestar] "change A, not B");
  - planted mistakes in copies of the C loop fail the autograd pin.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle.attention as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS = [[0, 3, 5, 9], [0, 9], [0, 1, 2, 3], [0, 7, 8, 20, 33]]


def _case(cu, H=2, d=16, seed=0):
    T = cu[-1]
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, d)) for _ in range(4)]


def _autograd(q, k, v, g, cu, causal):
    allow = torch.from_numpy(A.allow_matrix(cu, causal))
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    d = q.shape[-1]
    S = torch.einsum("ihc,jhc->hij", Q, K) / np.sqrt(d)
    S = S.masked_fill(~allow, float("-inf"))
    O = torch.einsum("hij,jhc->ihc", torch.softmax(S, dim=-1), V)
    (O * torch.from_numpy(g)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("cu", CUS)
@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_autograd(cu, causal):
    q, k, v, g = _case(cu)
    ours = A.attention_bwd(q, k, v, g, cu, causal)
    ref = _autograd(q, k, v, g, cu, causal)
    for a, b in zip(ours, ref):
        assert np.abs(a - b).max() < 1e-12


def test_matches_finite_differences_of_forward_oracle():
    cu = [0, 3, 5, 9]
    q, k, v, g = _case(cu, H=1, d=4, seed=5)
    dq, dk, dv = A.attention_bwd(q, k, v, g, cu, True)
    loss = lambda q_, k_, v_: float((A.attention_brute(q_, k_, v_, cu, True)[0] * g).sum())  # noqa: E731
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        for idx in [(0, 0, 1), (4, 0, 2), (8, 0, 3), (2, 0, 0)]:
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7, (which, idx, fd, grad[idx])


def test_closed_forms():
    cu = [0, 1, 4, 9]
    rng = np.random.default_rng(2)
    T, H, d = 9, 2, 8
    q, k, v, g = (rng.standard_normal((T, H, d)) for _ in range(4))
    dq, dk, dv = A.attention_bwd(q, k, v, g, cu, True)
    for s in (0, 1, 4):                 # first row of each segment sees one key
        assert np.all(dq[s] == 0.0)
    assert np.all(dk[0] == 0.0) and np.all(dv[0] == g[0])    # one-token segment
    # q = 0: uniform weights over the visible keys
    z = np.zeros_like(q)
    dq0, dk0, dv0 = A.attention_bwd(z, k, v, g, cu, True)
    assert np.all(dk0 == 0.0)
    want = np.zeros_like(dv0)
    for r in range(len(cu) - 1):
        s, e = cu[r], cu[r + 1]
        for j in range(s, e):
            for i in range(j, e):
                want[j] += g[i] / (i - s + 1)
    assert np.abs(dv0 - want).max() < 1e-13


def test_packed_equals_segment_alone():
    cu = [0, 7, 8, 20, 33]
    q, k, v, g = _case(cu, seed=9)
    packed = A.attention_bwd(q, k, v, g, cu, True)
    for r in range(len(cu) - 1):
        s, e = cu[r], cu[r + 1]
        alone = A.attention_bwd(q[s:e], k[s:e], v[s:e], g[s:e], [0, e - s], True)
        for a, b in zip(packed, alone):
            assert np.array_equal(a[s:e], b)


def test_restriction_to_heads_and_segments():
    cu = [0, 3, 5, 9]
    q, k, v, g = _case(cu)
    full = A.attention_bwd(q, k, v, g, cu, True)
    part = A.attention_bwd(q, k, v, g, cu, True, heads=[1], segments=[2])
    for a, b in zip(full, part):
        assert np.array_equal(a[5:9, 1], b[5:9, 1])
        assert np.isnan(b[0:5]).all() and np.isnan(b[:, 0]).all()


@pytest.mark.parametrize("old,new", [
    ("ds[j] = p[j] * (dp - D);", "ds[j] = p[j] * dp;"),                 # softmax Jacobian term dropped
    ("dqi[c] = acc * inv_sqrt_d;", "dqi[c] = acc;"),                    # scale dropped from dQ
    ("dv[j * ld + c] += p[j] * gi[c];", "dv[j * ld + c] += p[j] * qi[c];"),   # wrong operand in dV
    ("const int64_t j_end = causal ? i + 1 : n;", "const int64_t j_end = causal ? i : n;"),  # diagonal dropped
])
def test_planted_mistakes_are_caught(tmp_path, old, new):
    with open(os.path.join(ROOT, "oracle", "attn_oracle.c")) as f:
        src = f.read()
    assert old in src
    cfile = tmp_path / "bwd_mutant.c"
    cfile.write_text(src.replace(old, new, 1))
    so = tmp_path / "bwd_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(so), str(cfile), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    p = ctypes.c_void_p
    lib.oracle_attn_bwd_segment.argtypes = [p, p, p, p, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int64, ctypes.c_int32, p, p, p, p]
    cu = [0, 9]
    q, k, v, g = _case(cu, H=1, d=8, seed=4)
    outs = [np.empty_like(q) for _ in range(3)]
    scratch = np.empty(2 * 9 + 8)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    with np.errstate(all="ignore"):
        lib.oracle_attn_bwd_segment(ptr(q), ptr(k), ptr(v), ptr(g), 9, 8, 8, 1, *(ptr(o) for o in outs),
                                    ptr(scratch))
    ref = _autograd(q, k, v, g, cu, True)
    err = max(np.nan_to_num(np.abs(a - b), nan=np.inf).max() for a, b in zip(outs, ref))
    assert err > 1e-6
