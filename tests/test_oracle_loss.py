"""Pins of the packed cross-entropy oracle (CPU only).

The oracle is pinned to things other than itself:
  - the values printed on the pages (golden loss_examples.json): six targets
    for the nine-token pack; token average 2.5 vs sample average 2;
  - PyTorch's float64 cross_entropy (reduction "sum", ignore_index) on the
    same rows, and its internal-shift form with segment starts ignored, as
    the page writes it;
  - closed forms: uniform logits give log V per target; a two-class row
    [0, log(e^c - 1)] with label 0 gives exactly c; adding a constant to a row
    changes nothing; huge logits stay finite;
  - the gradient: central finite differences of the loss sum, rows that sum
    to zero, ignored rows that are zero, PyTorch autograd;
  - planted mistakes in copies of the oracle fail these pins.
"""

import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

import oracle.loss as L
import oracle.pack as P


def _case(T=40, V=17, seed=0, scale=3.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, V)) * scale
    return z


def _labels(lengths, V, seed=1):
    toks = np.random.default_rng(seed).integers(0, V, sum(lengths)).astype(np.int32)
    return P.pack_build(lengths, tokens=toks)


def test_nine_token_pack_has_six_targets(golden):
    case = golden("loss_examples.json")["nine_token_targets"]
    meta = _labels(case["lengths"], 50)
    z = _case(9, 50)
    out = L.packed_loss(z, meta["shifted_labels"], meta["cu_seqlens"])
    assert out["target_count"] == case["target_count"]
    assert out["seg_count"].tolist() == [L_ - 1 for L_ in case["lengths"]]


def test_token_vs_sample_average(golden):
    case = golden("loss_examples.json")["token_vs_sample_average"]
    # one row per target plus one ignored row closing each sample; two classes,
    # logits [0, log(e^c - 1)] and label 0, so each target's loss is exactly c
    rows, labels, cu = [], [], [0]
    for smp in case["samples"]:
        c = smp["loss_per_target"]
        for _ in range(smp["targets"]):
            rows.append([0.0, math.log(math.expm1(c))])
            labels.append(0)
        rows.append([0.0, 0.0])
        labels.append(L.IGNORE_INDEX)
        cu.append(len(labels))
    out = L.packed_loss(np.array(rows), np.array(labels), cu)
    assert out["seg_count"].tolist() == [s["targets"] for s in case["samples"]]
    assert abs(L.token_average(out["seg_loss"], out["seg_count"]) - case["token_average"]) < 1e-12
    assert abs(L.sample_average(out["seg_loss"], out["seg_count"]) - case["sample_average"]) < 1e-12


def test_matches_torch_cross_entropy_sum():
    lengths = [7, 1, 12, 5, 15]
    meta = _labels(lengths, 23)
    z = _case(sum(lengths), 23, seed=3)
    out = L.packed_loss(z, meta["shifted_labels"], meta["cu_seqlens"])
    lab = torch.from_numpy(meta["shifted_labels"].astype(np.int64))
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), lab, ignore_index=-100, reduction="sum")
    assert abs(out["loss_sum"] - ref.item()) < 1e-10
    assert out["target_count"] == int((lab != -100).sum())
    per = torch.nn.functional.cross_entropy(torch.from_numpy(z), lab, ignore_index=-100, reduction="none")
    assert np.abs(out["row_loss"] - per.numpy()).max() < 1e-12
    for r in range(len(lengths)):
        s, e = meta["cu_seqlens"][r], meta["cu_seqlens"][r + 1]
        assert abs(out["seg_loss"][r] - per[s:e].sum().item()) < 1e-12


def test_page_internal_shift_form_gives_the_same_sum():
    """The page's form: labels = tokens with each segment start ignored,
    logits[:-1] against labels[1:].  Same pairs as the pre-shifted labels."""
    lengths = [3, 2, 4]
    V = 31
    toks = np.random.default_rng(5).integers(0, V, 9)
    meta = P.pack_build(lengths, tokens=toks.astype(np.int32))
    z = _case(9, V, seed=6)
    ours = L.packed_loss(z, meta["shifted_labels"])
    lab = torch.from_numpy(toks.astype(np.int64)).clone()
    lab[torch.from_numpy(meta["cu_seqlens"][:-1].astype(np.int64))] = -100
    page = torch.nn.functional.cross_entropy(torch.from_numpy(z)[:-1], lab[1:], ignore_index=-100,
                                             reduction="sum")
    assert abs(ours["loss_sum"] - page.item()) < 1e-12
    assert ours["target_count"] == int((lab[1:] != -100).sum()) == 6


def test_closed_forms():
    V = 1000
    z = np.full((4, V), 0.37)
    out = L.packed_loss(z, np.array([0, 5, L.IGNORE_INDEX, 999]))
    assert np.allclose(out["row_loss"], [math.log(V), math.log(V), 0.0, math.log(V)], rtol=0, atol=1e-12)
    assert out["target_count"] == 3
    # a row shifted by a constant keeps its loss
    z = _case(6, 40, seed=8)
    lab = np.array([1, 2, 3, 4, 5, 6])
    a = L.packed_loss(z, lab)["row_loss"]
    b = L.packed_loss(z + np.arange(6)[:, None] * 1e3, lab)["row_loss"]
    assert np.abs(a - b).max() < 1e-9
    # huge logits stay finite: [1000, 0] -> loss 0 (label 0) or 1000 (label 1)
    out = L.packed_loss(np.array([[1000.0, 0.0], [1000.0, 0.0]]), np.array([0, 1]))
    assert abs(out["row_loss"][0] - math.log1p(math.exp(-1000.0))) < 1e-300
    assert abs(out["row_loss"][1] - 1000.0) < 1e-12


def test_bad_labels_flagged_and_skipped():
    z = _case(4, 10)
    out = L.packed_loss(z, np.array([3, 10, -1, L.IGNORE_INDEX]))
    assert out["err"] == L.ERR_LABEL
    assert out["target_count"] == 1
    assert out["row_loss"][1] == 0 and out["row_loss"][2] == 0


def test_gradient():
    lengths = [4, 1, 6]
    V = 9
    meta = _labels(lengths, V, seed=2)
    lab = meta["shifted_labels"]
    z = _case(sum(lengths), V, seed=4)
    g = L.loss_grad(z, lab, scale=0.5)
    # PyTorch autograd of the sum
    zt = torch.from_numpy(z).requires_grad_()
    torch.nn.functional.cross_entropy(zt, torch.from_numpy(lab.astype(np.int64)), ignore_index=-100,
                                      reduction="sum").backward()
    assert np.abs(g - 0.5 * zt.grad.numpy()).max() < 1e-14
    # rows sum to zero; ignored rows are zero
    assert np.abs(g.sum(axis=1)).max() < 1e-14
    assert (g[lab == L.IGNORE_INDEX] == 0).all()
    # central finite differences of the loss sum along random directions
    rng = np.random.default_rng(0)
    for _ in range(3):
        dz = rng.standard_normal(z.shape)
        h = 1e-6
        fd = (L.packed_loss(z + h * dz, lab)["loss_sum"] - L.packed_loss(z - h * dz, lab)["loss_sum"]) / (2 * h)
        assert abs(fd - (L.loss_grad(z, lab) * dz).sum()) < 1e-7


def test_bf16_bits_input():
    from workloads import f32_to_bf16_bits
    z = _case(5, 12, seed=9).astype(np.float32)
    bits = f32_to_bf16_bits(z)
    lab = np.array([0, 1, 2, 3, 4])
    exact = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert L.packed_loss(bits, lab)["loss_sum"] == L.packed_loss(exact, lab)["loss_sum"]


def _mutate(fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(L, fname)))
    assert old in src, (fname, old)
    ns = dict(vars(L))
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


@pytest.mark.parametrize("old,new", [
    ("lse[rows] - z[rows, labels[a + rows]]", "lse[rows] - z[rows, labels[a + rows] - 1]"),   # label off by one
    ("m + np.log(", "np.log("),                                                               # max not added back
    ("valid = (labels != ignore_index) & (labels >= 0)", "valid = (labels != labels + 1) & (labels >= -1000)"),  # ignored rows counted
])
def test_planted_mistakes_in_row_losses_are_caught(old, new):
    bad = _mutate("row_losses", old, new)
    lengths = [7, 1, 12, 5]
    meta = _labels(lengths, 23)
    z = _case(sum(lengths), 23, seed=3)
    lab = meta["shifted_labels"]
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(lab.astype(np.int64)),
                                            ignore_index=-100, reduction="none").numpy()
    try:
        loss, valid, _ = bad(z, lab)
    except IndexError:
        return                        # the mutant cannot even run on the pinned case
    with np.errstate(invalid="ignore"):
        assert not (np.abs(loss - ref).max() < 1e-10 and valid.sum() == (lab != -100).sum())


def test_planted_mistake_in_gradient_is_caught():
    bad = _mutate("loss_grad", "p[np.arange(rows.size), labels[rows]] -= 1.0", "p[np.arange(rows.size), labels[rows]] -= 0.0")
    z = _case(6, 7, seed=1)
    lab = np.array([0, 1, 2, -100, 4, 5])
    assert np.abs(bad(z, lab).sum(axis=1)).max() > 0.5


def test_planted_mistake_in_segment_sums_is_caught(golden):
    bad = _mutate("packed_loss", "seg_loss[r] = loss[s:e].sum()", "seg_loss[r] = loss[s:e - 1].sum()")
    case = golden("loss_examples.json")["token_vs_sample_average"]
    rows, labels, cu = [], [], [0]
    for smp in case["samples"]:
        for _ in range(smp["targets"]):
            rows.append([0.0, math.log(math.expm1(smp["loss_per_target"]))])
            labels.append(0)
        cu.append(len(labels))
    out = bad(np.array(rows), np.array(labels), cu)
    assert abs(L.token_average(out["seg_loss"], out["seg_count"]) - case["token_average"]) > 1e-3
