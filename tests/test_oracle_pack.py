"""Pins for the packing-metadata oracle (CPU only).

Each test checks the oracle against something other than its own formula:
values printed on the pages (tests/golden), a token-by-token concatenation
built the way the pages' pack builder builds it, closed-form counts, and
error cases the pages name.
"""

import numpy as np
import pytest

from oracle import pack as P
from workloads import EOS_ID, make_workload, token_ids


def test_cu_seqlens_printed_examples(golden):
    for case in golden("packing_examples.json")["cu_seqlens"]:
        out = P.pack_build(case["lengths"])
        assert out["error"] == 0
        assert out["cu_seqlens"].tolist() == case["cu_seqlens"], case["cite"]


def test_nine_token_segments_positions_max(golden):
    case = golden("packing_examples.json")["cu_seqlens"][1]
    out = P.pack_build(case["lengths"], tokens=np.arange(9))
    assert out["segment_ids"].tolist() == case["segment_ids"]
    assert out["position_ids"].tolist() == case["position_ids"]
    assert out["max_seqlen"] == case["max_seqlen"]          # 4, not the total 9
    assert int(out["cu_seqlens"][-1]) == case["total_tokens"]


def test_labels_m020_example(golden):
    case = golden("packing_examples.json")["labels"][0]
    samples = case["samples"]
    toks = [t for s in samples for t in s]
    out = P.pack_build([len(s) for s in samples], tokens=toks)
    want = [P.IGNORE_INDEX if x is None else x for x in case["pre_shifted_labels"]]
    assert out["shifted_labels"].tolist() == want, case["cite"]
    assert out["num_targets"] == case["num_targets"]
    assert out["loss_mask"].tolist() == [int(x is not None) for x in case["pre_shifted_labels"]]


def test_labels_charlestar_example_both_conventions(golden):
    """The page prints internal-shift labels (segment starts ignored, the loss
    shifts by one).  It states that this and pre-shifted targets (ignore on
    each segment's last position) are the same contract when not mixed: the
    pre-shifted labels are the internal-shift labels moved left by one."""
    case = golden("packing_examples.json")["labels"][1]
    samples = case["samples"]
    vocab = {name: i + 100 for i, name in enumerate(sorted({t for s in samples for t in s}))}
    toks = [vocab[t] for s in samples for t in s]
    internal = [P.IGNORE_INDEX if x is None else vocab[x] for x in case["internal_shift_labels"]]
    want = internal[1:] + [P.IGNORE_INDEX]
    out = P.pack_build([len(s) for s in samples], tokens=toks)
    assert out["shifted_labels"].tolist() == want
    assert out["num_targets"] == case["num_targets"] == sum(len(s) - 1 for s in samples)


def _concat_reference(samples, pad_flags):
    """Build ids/segment/position/labels by appending sample after sample, as
    the pages' pack builder does (position restarts from 0 for each sample;
    targets are the next token inside the sample)."""
    ids, seg, pos, lab = [], [], [], []
    for r, (s, pad) in enumerate(zip(samples, pad_flags)):
        ids += list(s)
        seg += [r] * len(s)
        pos += list(range(len(s)))
        lab += ([-100] * len(s)) if pad else (list(s[1:]) + [-100])
    return ids, seg, pos, lab


@pytest.mark.parametrize("name", ["tiny", "sft", "pretrain", "longctx", "short"])
def test_pack_build_against_concatenation(name):
    w = make_workload(name, scale="small")
    toks = token_ids(w)
    samples, start = [], 0
    for L in w.lengths.tolist():
        samples.append(toks[start:start + L].tolist())
        start += L
    ids, seg, pos, lab = _concat_reference(samples, w.is_pad.tolist())
    out = P.pack_build(w.lengths, tokens=toks, is_pad=w.is_pad)
    assert out["error"] == 0
    assert toks.tolist() == ids
    assert out["segment_ids"].tolist() == seg
    assert out["position_ids"].tolist() == pos
    assert out["shifted_labels"].tolist() == lab
    # closed form: every real sample of length L contributes L - 1 targets
    assert out["num_targets"] == int(sum(L - 1 for L, p in zip(w.lengths, w.is_pad) if not p))
    assert out["max_seqlen"] == int(w.lengths.max())


def test_pad_tail_is_own_segment_with_ignored_labels():
    """[compass] implementation notes: the pack builder pads the tail, gives it
    labels -100 everywhere and closes the prefix with the padded length."""
    w = make_workload("sft", scale="small")
    out = P.pack_build(w.lengths, tokens=token_ids(w), is_pad=w.is_pad)
    cu = out["cu_seqlens"]
    assert w.is_pad.sum() > 0
    for r in np.nonzero(w.is_pad)[0]:
        s, e = cu[r], cu[r + 1]
        assert (out["shifted_labels"][s:e] == P.IGNORE_INDEX).all()
        assert (out["loss_mask"][s:e] == 0).all()
    # every pack closes at a multiple of the capacity
    assert cu[-1] % 1024 == 0


def test_eos_targets_kept():
    """[charlestar] cross-boundary pairs: the in-sample 'x -> EOS' target stays;
    only the prediction from a sample's last token into the next sample goes."""
    w = make_workload("tiny")
    toks = token_ids(w)
    out = P.pack_build(w.lengths, tokens=toks)
    cu = out["cu_seqlens"]
    for r in range(w.nseg):
        last = cu[r + 1] - 1
        assert toks[last] == EOS_ID
        assert out["shifted_labels"][last - 1] == EOS_ID   # x -> EOS kept
        assert out["shifted_labels"][last] == P.IGNORE_INDEX  # EOS -> next sample dropped


def test_validate_bad_prefix_detected(golden):
    case = golden("packing_examples.json")["bad_prefix"]
    cu = case["cu_seqlens"]
    # the shape and dtype look right and the array is a valid prefix sum ...
    assert P.validate_cu(cu, 9, 4) == 0
    # ... only the lengths it should come from expose it
    assert P.validate_cu(cu, 9, 4, lengths=case["lengths"]) == P.ERR_MISMATCH


@pytest.mark.parametrize("cu,T,maxlen,bits", [
    ([0, 3, 5, 9], 9, 4, 0),
    ([1, 3, 5, 9], 9, 4, P.ERR_CU0),
    ([0, 3, 3, 9], 9, 6, P.ERR_NOT_INCREASING),
    ([0, 5, 3, 9], 9, 6, P.ERR_NOT_INCREASING),
    ([0, 3, 5, 8], 9, 4, P.ERR_TOTAL),
    ([0, 3, 5, 9], 9, 3, P.ERR_MAXSEQ),
    ([0, 9], 9, 9, 0),
])
def test_validate_bits(cu, T, maxlen, bits):
    assert P.validate_cu(cu, T, maxlen) == bits


def test_pack_build_rejects_nonpositive_lengths():
    assert P.pack_build([3, 0, 2])["error"] & P.ERR_LENGTH
    assert P.pack_build([3, -1, 2])["error"] & P.ERR_LENGTH
    assert P.pack_build([2**30, 2**30, 2**30])["error"] & P.ERR_RANGE
