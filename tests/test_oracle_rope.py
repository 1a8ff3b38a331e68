"""Pins for the RoPE oracle (CPU only): closed forms and invariants."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import pack as P
from oracle import rope as R
from workloads import make_workload, qkv_bits


def test_bf16_rounding_against_exact_nearest():
    """f64 -> bf16 rounding checked against exact rational arithmetic: pick the
    nearer of the two bf16 neighbours, ties to the even mantissa."""
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.standard_normal(3000) * 4,
                         # exact ties and near-ties between bf16 neighbours
                         (1 + (np.arange(200) * 2 + 1) / 256.0),
                         (1 + (np.arange(200) * 2 + 1) / 256.0) * (1 + 1e-15)])
    got = R.f64_to_bf16_bits(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        fx = Fraction(x)
        e = math.frexp(abs(x))[1] - 1            # |x| in [2^e, 2^(e+1))
        ulp = Fraction(2) ** (e - 7)
        lo = (abs(fx) // ulp) * ulp
        hi = lo + ulp
        dl, dh = abs(fx) - lo, hi - abs(fx)
        if dl < dh or (dl == dh and (lo / ulp) % 2 == 0):
            pick = lo
        else:
            pick = hi
        pick = -pick if x < 0 else pick
        u = np.asarray([g], np.uint32) << np.uint32(16)
        gv = float(u.view(np.float32)[0])
        assert Fraction(gv) == pick, (x, gv, float(pick))


def test_freqs_closed_form():
    f = R.rope_freqs(128, 10000.0)
    assert f.dtype == np.float32 and f.shape == (64,)
    assert f[0] == 1.0
    assert f[32] == np.float32(0.01)      # 10000^(-64/128) = 1/100
    assert np.all(np.diff(f.astype(np.float64)) < 0)
    assert abs(float(f[-1]) - 10000.0 ** (-126 / 128)) < 1e-9


def test_rotation_matches_complex_multiplication():
    """Rotate-half pair (x_j, x_{j+d/2}) read as the complex number
    x_j + i x_{j+d/2}; rotation by theta is multiplication by e^{i theta}."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 16))
    theta = rng.uniform(-50, 50, (5, 8)).astype(np.float32)
    y = R.rotate_f64(x, theta)
    z = (x[..., :8] + 1j * x[..., 8:]) * np.exp(1j * theta.astype(np.float64))[:, None, :]
    np.testing.assert_allclose(y[..., :8], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., 8:], z.imag, rtol=0, atol=1e-13)
    # a rotation keeps the norm of every pair
    n0 = x[..., :8] ** 2 + x[..., 8:] ** 2
    n1 = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n0, n1, rtol=1e-13)


def test_hand_value_position_one():
    """p = 1, j = 0: theta = 1 rad exactly; y_0 = x_0 cos 1 - x_{d/2} sin 1."""
    d = 8
    x = np.zeros((2, 1, d), np.float64)
    x[1, 0, 0], x[1, 0, 4] = 1.0, 2.0
    bits = R.f64_to_bf16_bits(x)
    out = R.rope_apply(bits, [0, 2])
    y = R.bf16_bits_to_f64(out)
    assert y[1, 0, 0] == R.bf16_bits_to_f64(R.f64_to_bf16_bits(np.array([math.cos(1) - 2 * math.sin(1)])))[0]
    assert y[1, 0, 4] == R.bf16_bits_to_f64(R.f64_to_bf16_bits(np.array([2 * math.cos(1) + math.sin(1)])))[0]
    assert (out[0] == bits[0]).all()


def test_position_zero_is_identity_per_segment():
    w = make_workload("sft", scale="small")
    x = qkv_bits(w, "q")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    y = R.rope_apply(x, cu)
    starts = cu[:-1]
    assert (y[starts] == x[starts]).all()          # p = 0 at every segment start, bit-exact
    assert (y[starts + 1] != x[starts + 1]).any()  # and not elsewhere


def test_segment_reset_equals_standalone():
    """RoPE of a segment inside the pack equals RoPE of that segment alone."""
    w = make_workload("longctx", scale="small")
    x = qkv_bits(w, "k")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    y = R.rope_apply(x, cu)
    for r in range(w.nseg):
        s, e = int(cu[r]), int(cu[r + 1])
        alone = R.rope_apply(x[s:e], [0, e - s])
        assert (alone == y[s:e]).all()


def test_positions_continued_differs():
    """Not resetting positions (one whole-pack segment) changes later segments."""
    w = make_workload("tiny")
    x = qkv_bits(w, "q")
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    reset = R.rope_apply(x, cu)
    cont = R.rope_apply(x, [0, w.total_tokens])
    assert (reset[:3] == cont[:3]).all()
    assert (reset[3:] != cont[3:]).any()


@pytest.mark.parametrize("c", [1, 7, 400, 12345])
def test_shift_invariance(c):
    """(R(m+c)q)^T (R(n+c)k) = q^T R(n-m) k with exact double angles."""
    rng = np.random.default_rng(c)
    d = 64
    f = R.rope_freqs(d).astype(np.float64)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for m, n in [(0, 0), (3, 1), (17, 40), (250, 2)]:
        a = R.rotate_f64(q, ((m + c) * f)[None]).ravel() @ R.rotate_f64(k, ((n + c) * f)[None]).ravel()
        b = q.ravel() @ R.rotate_f64(k, ((n - m) * f)[None]).ravel()
        assert abs(a - b) <= 1e-9 * max(1.0, abs(b))


def test_interleaved_matches_complex_multiplication():
    """Interleaved pair (x_{2j}, x_{2j+1}) as x_{2j} + i x_{2j+1}, turned by
    e^{i theta_j} (the RoFormer complex form)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 16))
    theta = rng.uniform(-50, 50, (5, 8)).astype(np.float32)
    y = R.rotate_interleaved_f64(x, theta)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * theta.astype(np.float64))[:, None, :]
    np.testing.assert_allclose(y[..., 0::2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], z.imag, rtol=0, atol=1e-13)


def test_interleaved_is_rotate_half_under_a_permutation():
    """Moving element 2j to j and 2j+1 to j + d/2 turns the interleaved pairing
    into the rotate-half one: interleaved(x) = P^-1 rotate_half(P x)."""
    w = make_workload("sft", scale="small")
    x = qkv_bits(w, "k")
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])     # new index -> old index
    cu = P.pack_build(w.lengths)["cu_seqlens"]
    a = R.rope_apply(x, cu, interleaved=True)
    b = R.rope_apply(np.ascontiguousarray(x[..., perm]), cu)
    inv = np.argsort(perm)
    assert (a == b[..., inv]).all()
    assert (a != R.rope_apply(x, cu)).any()
    starts = cu[:-1]
    assert (a[starts] == x[starts]).all()          # p = 0 stays the identity


def test_interleaved_shift_invariance():
    rng = np.random.default_rng(5)
    d = 32
    f = R.rope_freqs(d).astype(np.float64)
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    for m, n, c in [(0, 0, 9), (3, 1, 100), (17, 40, 5)]:
        rot = R.rotate_interleaved_f64
        a = rot(q, ((m + c) * f)[None]).ravel() @ rot(k, ((n + c) * f)[None]).ravel()
        b = q.ravel() @ rot(k, ((n - m) * f)[None]).ravel()
        assert abs(a - b) <= 1e-9 * max(1.0, abs(b))


def test_f16_rounding_against_exact_nearest():
    """f64 -> fp16 rounding against exact rationals: the nearer neighbour on the
    fp16 grid (11 significant bits; a fixed 2^-24 spacing below 2^-14), ties to
    the even last bit, including subnormals and exact ties."""
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.standard_normal(2000) * 4,
                         rng.standard_normal(500) * 1e-6,                       # fp16 subnormal range
                         1 + (np.arange(200) * 2 + 1) / 2048.0,                 # exact ties at 1..2
                         (np.arange(1, 101) * 2 + 1) * 2.0 ** -25])            # exact subnormal ties
    got = R.f64_to_f16_bits(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        fx = abs(Fraction(x))
        e = max(math.frexp(abs(x))[1] - 1, -14) if x != 0 else -14
        ulp = Fraction(2) ** (e - 10)
        lo = (fx // ulp) * ulp
        hi = lo + ulp
        dl, dh = fx - lo, hi - fx
        pick = lo if (dl < dh or (dl == dh and (lo / ulp) % 2 == 0)) else hi
        pick = -pick if x < 0 else pick
        gv = float(np.asarray([g], np.uint16).view(np.float16)[0])
        assert Fraction(gv) == pick, (x, gv, float(pick))


def test_f16_rope_matches_the_same_rotation_rounded_to_fp16():
    """The fp16 path rotates the fp16 input values and rounds once to fp16;
    position 0 is the identity."""
    rng = np.random.default_rng(9)
    x16 = (rng.standard_normal((20, 2, 16)) * 3).astype(np.float16)
    bits = x16.view(np.uint16)
    cu = np.array([0, 7, 20])
    y = R.rope_apply(bits, cu, 500.0, f16=True)
    theta = R.rope_angles(P.positions_from_cu(cu), 16, 500.0)
    want = R.rotate_f64(x16.astype(np.float64), theta).astype(np.float16).view(np.uint16)
    assert (y == want).all()
    assert (y[[0, 7]] == bits[[0, 7]]).all()
