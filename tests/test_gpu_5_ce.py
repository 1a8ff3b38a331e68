"""GPU parity for the packed cross-entropy (loss sum, target count, per-row and
per-segment values, fused gradient) against the fp64 oracle (oracle.loss).

Integers (target counts) must match exactly.  Floating-point values are
compared with first-order bounds derived from the kernel's fp32 arithmetic
(see ``row_bound`` / ``grad_bound``); sums run in fp64 in the kernel, so their
bound is the sum of the row bounds.  The bf16 gradient must equal the RNE
rounding of the fp32 gradient bit for bit (the two differ only in the store),
and the in-place gradient must equal the out-of-place one.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev_i32, host_bits, say
from oracle import loss as L
from oracle import pack as P
from workloads import f32_to_bf16_bits, logits_bits, make_workload

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _f64(bits):
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def row_bound(z, ref_loss):
    """|kernel row loss - fp64 loss| for one row set, first order in fp32 units:
    the exponent arguments fma(x, log2 e, -max log2 e) carry 2^-24 (|max| +
    |x - max|) log2 e each (only terms within 40 of the max matter), exp2 and
    log2 one ulp, the fp32 sum of V terms (V / 256 sequential per thread plus
    the chunk rescales and a 256-way merge) (V / 256 + 24) 2^-24, and the two
    final roundings |lse| and |loss| 2^-24."""
    z = np.asarray(z, np.float64)
    V = z.shape[1]
    m = z.max(axis=1)
    spread = np.minimum(m - z.min(axis=1), 40.0)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return U32 * (1.5 * (np.abs(m) + spread) + 4 + (V / 256 + 24) + 2 * np.abs(lse) + np.abs(ref_loss))


def grad_bound(z, labels, scale):
    """Elementwise bound of the fp32 gradient scale (p - onehot): the argument
    fma(x - max, log2 e, -log2 s) carries 2^-24 (2 |x - max| log2 e + |arg|)
    plus the error of log2 s (the sum's (V / 256 + 24) 2^-24 relative error),
    exp2 one ulp; then two fp32 roundings of (p - onehot) and the product.
    Values below 2^-126 may be flushed (|scale| 2^-126)."""
    z = np.asarray(z, np.float64)
    V = z.shape[1]
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    p = np.exp(z - lse)
    arg = (z - lse) / np.log(2.0)
    rel = U32 * (2 * np.abs(z - m) * 1.4427 + np.abs(arg) + 2 * (V / 256 + 24) + 2 + 2 * np.abs(lse) * 1.4427)
    onehot = np.zeros_like(z)
    ok = (labels >= 0) & (labels < V)
    onehot[np.nonzero(ok)[0], labels[ok]] = 1.0
    b = abs(scale) * (p * rel + 2 * U32 * np.abs(p - onehot) + 2.0 ** -126)
    b[~ok] = 0.0
    return b


def _dev_logits(bits, dtype=torch.bfloat16):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return t if dtype == torch.bfloat16 else t.float()


def _check_loss(out, ref, z, cu=None):
    rl = out["row_loss"].cpu().numpy().astype(np.float64)
    bound = row_bound(z, ref["row_loss"])
    err = np.abs(rl - ref["row_loss"])
    ratio = float((err / bound).max())
    s = float(out["loss_sum"].item())
    rep = {"rows": rl.size, "max_row_err": float(err.max()), "max_err_over_bound": ratio,
           "loss_sum": s, "ref": ref["loss_sum"], "sum_err": abs(s - ref["loss_sum"]),
           "count": int(out["target_count"].item()), "ref_count": ref["target_count"]}
    say("    ce parity", rep)
    assert ratio <= 1.0, rep
    assert rep["count"] == ref["target_count"]
    assert abs(s - ref["loss_sum"]) <= bound[ref["valid"]].sum() + 1e-9 * abs(ref["loss_sum"])
    # the fp64 sum of the row losses the kernel wrote, in any order, to rounding
    assert abs(s - rl.sum()) <= 1e-12 * max(1.0, np.abs(rl).sum())
    if cu is not None:
        sl, sc = out["seg_loss"].cpu().numpy(), out["seg_count"].cpu().numpy()
        assert (sc == ref["seg_count"]).all()
        for r in range(len(cu) - 1):
            a, b = int(cu[r]), int(cu[r + 1])
            assert abs(sl[r] - ref["seg_loss"][r]) <= bound[a:b][ref["valid"][a:b]].sum() + 1e-12
    return rep


@pytest.mark.parametrize("name", ["tiny", "sft", "pretrain", "short"])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
def test_small_workloads_every_row(pvc, name, in_dtype):
    w = make_workload(name, scale="small")
    V = 32000
    T = w.total_tokens
    say(f"  ce small {name} {in_dtype}: T={T} V={V} nseg={w.nseg}")
    bits = logits_bits(w, V)
    meta = P.pack_build(w.lengths, w.tokens(), w.is_pad)
    lab = meta["shifted_labels"]
    cu = meta["cu_seqlens"]
    out = pvc.packed_ce_loss(_dev_logits(bits, in_dtype), dev_i32(lab), dev_i32(cu), row_loss=True,
                             segments=True)
    torch.cuda.synchronize()
    assert int(out["dev_error"].item()) == 0
    ref = L.packed_loss(bits, lab, cu)
    _check_loss(out, ref, _f64(bits), cu)


@pytest.mark.parametrize("V,ld", [(1, 1), (7, 7), (1001, 1001), (1001, 1003), (4096, 4104)])
def test_odd_vocab_and_strided_rows(pvc, V, ld):
    """Vocabularies that are not a multiple of 8 and row strides whose starts
    are not 16-byte aligned take the one-value-at-a-time path (or its tail)."""
    T = 257
    rng = np.random.default_rng(V + ld)
    bits = f32_to_bf16_bits(rng.standard_normal((T, ld), dtype=np.float32) * 3)
    lab = rng.integers(0, V, T).astype(np.int32)
    lab[::5] = -100
    say(f"  ce V={V} ld={ld}")
    full = _dev_logits(bits)
    out = pvc.packed_ce_loss(full[:, :V], dev_i32(lab), row_loss=True)
    torch.cuda.synchronize()
    ref = L.packed_loss(bits[:, :V], lab)
    _check_loss(out, ref, _f64(bits[:, :V]))
    if V == 1:
        assert (out["row_loss"].cpu() == 0).all()     # one class: log-sum-exp equals the logit


def test_gradient(pvc):
    w = make_workload("sft", scale="small")
    V, T = 32000, 300
    bits = logits_bits(w, V, rows=T)
    lab = P.pack_build([120, 1, 79, 100], np.random.default_rng(2).integers(3, V, T).astype(np.int32))["shifted_labels"]
    scale = float(np.float32(1.0 / 296))          # exact in fp32, as the kernel takes it
    say(f"  ce gradient T={T} V={V}")
    z = _dev_logits(bits)
    o32 = pvc.packed_ce_loss(z, dev_i32(lab), grad="new", grad_dtype=torch.float32, grad_scale=scale,
                             row_loss=True)
    o16 = pvc.packed_ce_loss(z, dev_i32(lab), grad="new", grad_scale=scale)
    zin = z.clone()
    oin = pvc.packed_ce_loss(zin, dev_i32(lab), grad="inplace", grad_scale=scale)
    torch.cuda.synchronize()
    g = o32["grad"].cpu().numpy().astype(np.float64)
    ref = L.loss_grad(bits, lab, scale)
    bnd = grad_bound(_f64(bits), lab, scale)
    err = np.abs(g - ref)
    say(f"    grad max err {err.max():.3e}, max err / bound {(err / np.maximum(bnd, 1e-300)).max():.3f}")
    assert (err <= bnd).all()
    assert (g[lab == -100] == 0).all()
    rne = host_bits(o32["grad"].to(torch.bfloat16))
    assert (rne == host_bits(o16["grad"])).all()
    assert (host_bits(zin) == host_bits(o16["grad"])).all()
    # the loss is the same with and without the gradient, and in place
    assert o32["loss_sum"].item() == o16["loss_sum"].item() == oin["loss_sum"].item()
    _check_loss(o32, L.packed_loss(bits, lab), _f64(bits))


def test_bad_labels_are_flagged_and_skipped(pvc):
    T, V = 64, 500
    rng = np.random.default_rng(3)
    bits = f32_to_bf16_bits(rng.standard_normal((T, V), dtype=np.float32))
    lab = rng.integers(0, V, T).astype(np.int32)
    lab[3], lab[10], lab[20] = V, -1, -100
    out = pvc.packed_ce_loss(_dev_logits(bits), dev_i32(lab), row_loss=True)
    torch.cuda.synchronize()
    ref = L.packed_loss(bits, lab)
    assert int(out["dev_error"].item()) == ref["err"] == L.ERR_LABEL
    _check_loss(out, ref, _f64(bits))


def test_ignore_index_inside_the_vocabulary(pvc):
    """An ignore index that is itself a class id (7 here) still marks its rows
    as ignored: no loss, no count, no gradient, as pack_build's loss mask
    (label != ignore index) and the oracle read it; per-segment counts too."""
    T, V, IGN = 200, 1001, 7
    rng = np.random.default_rng(9)
    bits = f32_to_bf16_bits(rng.standard_normal((T, V), dtype=np.float32) * 2)
    lab = rng.integers(0, V, T).astype(np.int32)
    lab[::4] = IGN
    lab[5] = -100                   # another class-free label: not a target, flagged
    cu = np.array([0, 50, 51, 130, 200], np.int32)
    scale = float(np.float32(1.0 / 128))
    out = pvc.packed_ce_loss(_dev_logits(bits), dev_i32(lab), dev_i32(cu), ignore_index=IGN, row_loss=True,
                             segments=True, grad="new", grad_dtype=torch.float32, grad_scale=scale)
    torch.cuda.synchronize()
    ref = L.packed_loss(bits, lab, cu, ignore_index=IGN)
    assert int(out["dev_error"].item()) == ref["err"] == L.ERR_LABEL
    assert int(out["target_count"].item()) == ref["target_count"] == int(((lab != IGN) & (lab >= 0)).sum())
    rl = out["row_loss"].cpu().numpy()
    assert (rl[lab == IGN] == 0).all()
    _check_loss(out, ref, _f64(bits), cu)
    g = out["grad"].cpu().numpy().astype(np.float64)
    gref = L.loss_grad(bits, lab, scale, ignore_index=IGN)
    bnd = grad_bound(_f64(bits), lab, scale)
    bnd[lab == IGN] = 0.0
    assert (g[lab == IGN] == 0).all()
    assert (np.abs(g - gref) <= bnd).all()


def test_large_logits_stay_finite(pvc):
    T, V = 16, 256
    rng = np.random.default_rng(4)
    z = rng.standard_normal((T, V)).astype(np.float32) * 3000
    bits = f32_to_bf16_bits(z)
    lab = rng.integers(0, V, T).astype(np.int32)
    out = pvc.packed_ce_loss(_dev_logits(bits), dev_i32(lab), row_loss=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out["row_loss"]).all()
    _check_loss(out, L.packed_loss(bits, lab), _f64(bits))


def test_deterministic(pvc):
    w = make_workload("pretrain", scale="small")
    V = 32000
    bits = logits_bits(w, V)
    meta = P.pack_build(w.lengths, w.tokens())
    z, lab, cu = _dev_logits(bits), dev_i32(meta["shifted_labels"]), dev_i32(meta["cu_seqlens"])
    runs = [pvc.packed_ce_loss(z, lab, cu, segments=True) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert r["loss_sum"].item() == runs[0]["loss_sum"].item()
        assert torch.equal(r["seg_loss"], runs[0]["seg_loss"])


def test_full_size_sampled_rows(pvc):
    """The benchmark's configuration (SFT packs, 32,768 rows x 32,000 logits,
    2 GiB of bf16 drawn on the device from a seeded generator): every row's
    target status and the count exactly, sampled rows against the oracle, the
    loss sum against the kernel's own row losses."""
    w = make_workload("sft")
    V, T = 32000, w.total_tokens
    say(f"  ce full sft T={T} V={V}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    z = (torch.randn((T, V), generator=gen, device="cuda", dtype=torch.float32) * 2).to(torch.bfloat16)
    meta = P.pack_build(w.lengths, w.tokens(), w.is_pad)
    lab = meta["shifted_labels"]
    out = pvc.packed_ce_loss(z, dev_i32(lab), dev_i32(meta["cu_seqlens"]), row_loss=True, segments=True)
    torch.cuda.synchronize()
    assert int(out["dev_error"].item()) == 0
    assert int(out["target_count"].item()) == meta["num_targets"]
    cu = meta["cu_seqlens"]
    want = np.array([(lab[cu[r]:cu[r + 1]] != L.IGNORE_INDEX).sum() for r in range(len(cu) - 1)])
    assert (out["seg_count"].cpu().numpy() == want).all()
    rows = np.unique(np.concatenate([meta["cu_seqlens"][1:] - 1, meta["cu_seqlens"][:-1],
                                     np.random.default_rng(1).integers(0, T, 256)]))
    rows = rows[rows < T]
    zb = host_bits(z[torch.from_numpy(rows).cuda()])
    ref = L.packed_loss(zb, lab[rows])
    rl = out["row_loss"].cpu().numpy().astype(np.float64)
    bound = row_bound(_f64(zb), ref["row_loss"])
    err = np.abs(rl[rows] - ref["row_loss"])
    say(f"    sampled rows {rows.size}: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    s = float(out["loss_sum"].item())
    assert abs(s - rl.sum()) <= 1e-12 * np.abs(rl).sum()
