"""Planted mistakes in copies of the oracle must fail a pin (CPU only).

Each case takes the source of an oracle function (Python or the C loop),
plants one plausible mistake (a dropped shift, a wrong sign, an off-by-one in
the mask, a wrong scale), rebuilds the copy and checks that the pin written
for that function now fails.  The oracle on disk is never modified.
"""

import ctypes
import inspect
import os
import subprocess
import textwrap

import numpy as np
import pytest
import torch

import oracle.attention as A
import oracle.pack as P
import oracle.rope as R
from oracle.rope import bf16_bits_to_f64, f64_to_bf16_bits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mutate(module, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, fname)))
    assert old in src, (fname, old)
    ns = dict(vars(module))
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


def test_label_shift_dropped_is_caught(golden):
    bad = _mutate(P, "pack_build", "tokens[s + 1:e]", "tokens[s:e - 1]")
    case = golden("packing_examples.json")["labels"][0]
    toks = [t for s in case["samples"] for t in s]
    want = [P.IGNORE_INDEX if x is None else x for x in case["pre_shifted_labels"]]
    assert bad([3, 2], tokens=toks)["shifted_labels"].tolist() != want
    assert P.pack_build([3, 2], tokens=toks)["shifted_labels"].tolist() == want


def test_positions_not_reset_is_caught(golden):
    bad = _mutate(P, "pack_build", "np.arange(e - s, dtype=np.int32)", "np.arange(s, e, dtype=np.int32)")
    case = golden("packing_examples.json")["cu_seqlens"][1]
    assert bad(case["lengths"])["position_ids"].tolist() != case["position_ids"]


def test_rotation_sign_is_caught():
    bad = _mutate(R, "rotate_f64", "x1 * c - x2 * s", "x1 * c + x2 * s")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 2, 16))
    theta = rng.uniform(-5, 5, (3, 8)).astype(np.float32)
    z = (x[..., :8] + 1j * x[..., 8:]) * np.exp(1j * theta.astype(np.float64))[:, None, :]
    assert np.abs(bad(x, theta)[..., :8] - z.real).max() > 1e-3
    assert np.abs(R.rotate_f64(x, theta)[..., :8] - z.real).max() < 1e-13


def test_frequency_exponent_is_caught():
    bad = _mutate(R, "rope_freqs", "-2.0 * j / head_dim", "-1.0 * j / head_dim")
    assert bad(128)[32] != np.float32(0.01)


def test_mask_off_by_one_is_caught():
    bad = _mutate(A, "allow_matrix", "j <= i", "j < i")
    assert bad([0, 3, 5, 9]).sum() != 19
    assert A.allow_matrix([0, 3, 5, 9]).sum() == 19


def _sdpa_case(seed=3):
    lengths = [3, 2, 4, 7]
    T = sum(lengths)
    rng = np.random.default_rng(seed)
    q, k, v = (f64_to_bf16_bits(rng.standard_normal((T, 2, 32))) for _ in range(3))
    cu = np.asarray(P.pack_build(lengths)["cu_seqlens"], np.int32)
    allow = A.allow_matrix(cu)
    Q, K, V = (torch.from_numpy(bf16_bits_to_f64(x)).permute(1, 0, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(allow))
    return q, k, v, cu, ref.permute(1, 0, 2).numpy()


def test_brute_scale_is_caught():
    bad = _mutate(A, "attention_brute", "/ np.sqrt(d)", "/ d")
    q, k, v, cu, ref = _sdpa_case()
    assert np.abs(bad(q, k, v, cu)[0] - ref).max() > 1e-3


def _build_c_mutant(tmp_path, old, new, name="mutant"):
    with open(os.path.join(ROOT, "oracle", "attn_oracle.c")) as f:
        src = f.read()
    assert old in src
    cfile = tmp_path / f"{name}.c"
    cfile.write_text(src.replace(old, new, 1))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(so), str(cfile), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_attn_rows.restype = ctypes.c_int
    return lib


def _run_c(lib, q, k, v, cu):
    T, H, d = q.shape
    rows = np.arange(T, dtype=np.int64)
    out = np.empty((T, H, d))
    lse = np.empty((T, H))
    scratch = np.empty(T)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    lib.oracle_attn_rows(p(q), p(k), p(v), p(cu), ctypes.c_int32(cu.shape[0] - 1),
                         ctypes.c_int32(H), ctypes.c_int32(d), ctypes.c_int32(1), p(rows),
                         ctypes.c_int64(T), p(out), p(lse), p(scratch))
    return out


@pytest.mark.parametrize("old,new", [
    ("causal ? i + 1 : ", "causal ? i : "),            # diagonal dropped from the mask
    ("const double s = dot * inv_sqrt_d;", "const double s = dot;"),   # scale dropped
    ("(j * heads + h)", "(h * heads + j)"),              # transposed head/token index
    ("oi[c] /= denom;", "oi[c] /= denom + 1.0;"),        # wrong normaliser
])
def test_c_oracle_mutants_are_caught(tmp_path, old, new):
    q, k, v, cu, ref = _sdpa_case()
    lib = _build_c_mutant(tmp_path, old, new)
    with np.errstate(all="ignore"):
        out = _run_c(lib, q, k, v, cu)
    err = np.nan_to_num(np.abs(out - ref), nan=np.inf).max()
    assert err > 1e-6
    good = _build_c_mutant(tmp_path, "/* scores of the allowed keys", "/* scores of the allowed keys", "unmutated")
    assert np.abs(_run_c(good, q, k, v, cu) - ref).max() < 1e-12


def test_interleaved_pair_swap_is_caught():
    bad = _mutate(R, "rotate_interleaved_f64", "x1, x2 = x[..., 0::2], x[..., 1::2]",
                  "x1, x2 = x[..., 1::2], x[..., 0::2]")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 2, 16))
    theta = rng.uniform(-5, 5, (3, 8)).astype(np.float32)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * theta.astype(np.float64))[:, None, :]
    assert np.abs(bad(x, theta)[..., 0::2] - z.real).max() > 1e-3
    assert np.abs(R.rotate_interleaved_f64(x, theta)[..., 0::2] - z.real).max() < 1e-13
