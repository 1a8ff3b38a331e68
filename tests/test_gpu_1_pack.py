"""GPU parity for pack_build and validate_cu_seqlens: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

from gpu_util import dev_i32, say
from oracle import pack as P
from workloads import CONFIG_NAMES, make_workload, token_ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _run_pack(pvc, lengths, tokens, is_pad, T=None):
    lt = dev_i32(lengths)
    tt = dev_i32(tokens) if tokens is not None else None
    pt = torch.from_numpy(np.asarray(is_pad, np.uint8)).cuda() if is_pad is not None else None
    out = pvc.pack_build(lt, tt, pt, total_tokens=T)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _compare(got, ref):
    assert got["dev_error"][0] == ref["error"] == 0
    assert (got["cu_seqlens"] == ref["cu_seqlens"]).all()
    assert got["max_seqlen"][0] == ref["max_seqlen"]
    for key in ("segment_ids", "position_ids", "shifted_labels", "loss_mask"):
        assert (got[key] == ref[key]).all(), key
    assert got["num_targets"][0] == ref["num_targets"]


def test_nine_token_example(pvc, golden):
    case = golden("packing_examples.json")["cu_seqlens"][1]
    say("  pack_build nine-token example")
    toks = np.arange(100, 109, dtype=np.int32)
    got = _run_pack(pvc, case["lengths"], toks, None)
    assert got["cu_seqlens"].tolist() == case["cu_seqlens"]
    assert got["segment_ids"].tolist() == case["segment_ids"]
    assert got["position_ids"].tolist() == case["position_ids"]
    assert got["max_seqlen"][0] == case["max_seqlen"]


def test_labels_m020_example(pvc, golden):
    case = golden("packing_examples.json")["labels"][0]
    toks = np.asarray([t for s in case["samples"] for t in s], np.int32)
    got = _run_pack(pvc, [3, 2], toks, None)
    want = [-100 if x is None else x for x in case["pre_shifted_labels"]]
    assert got["shifted_labels"].tolist() == want
    assert got["num_targets"][0] == case["num_targets"]


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_workloads_full_size(pvc, name):
    w = make_workload(name)
    say(f"  pack_build {name}: T={w.total_tokens} nseg={w.nseg}")
    toks = token_ids(w)
    got = _run_pack(pvc, w.lengths, toks, w.is_pad)
    _compare(got, P.pack_build(w.lengths, toks, w.is_pad))


def test_many_segments_multi_chunk_scan(pvc):
    """More than 8192 segments exercises the reduce / top-scan / apply path."""
    w = make_workload("short", total=1 << 20)
    assert w.nseg > 8192 * 1.5
    say(f"  pack_build multi-chunk: T={w.total_tokens} nseg={w.nseg}")
    toks = token_ids(w)
    got = _run_pack(pvc, w.lengths, toks, w.is_pad)
    _compare(got, P.pack_build(w.lengths, toks, w.is_pad))


@pytest.mark.parametrize("total,lo,hi", [((1 << 21) + 777, 8, 128), ((1 << 21) + 5, 1, 3), ((1 << 21) + 1, 1500, 6000)])
def test_large_buffer_block_map(pvc, total, lo, hi):
    """Above 2^20 tokens the scan writes, for every 2048-token block of the
    per-token pass, the segment its first token lies in (the workspace's
    block map); segments shorter than a 4-token group, and longer than a
    block, against the oracle bit for bit."""
    w = make_workload("short", total=total, lo=lo, hi=hi)
    say(f"  pack_build block map: T={w.total_tokens} nseg={w.nseg} lengths [{lo}, {hi}]")
    toks = token_ids(w)
    got = _run_pack(pvc, w.lengths, toks, w.is_pad)
    _compare(got, P.pack_build(w.lengths, toks, w.is_pad))


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_pack_tokens_on_given_cu(pvc, name):
    """The per-token pass alone, on pack_build's cu_seqlens (computed without
    its own per-token pass) and on a second stream: the same bits as the
    oracle, and num_targets cleared by the call (the word starts dirty)."""
    w = make_workload(name)
    toks = token_ids(w)
    ref = P.pack_build(w.lengths, toks, w.is_pad)
    side = torch.cuda.Stream()
    meta = pvc.pack_build(dev_i32(w.lengths), total_tokens=w.total_tokens, per_token=False)
    assert "segment_ids" not in meta and "shifted_labels" not in meta
    done = torch.cuda.Event()
    done.record()
    side.wait_event(done)
    pt = torch.from_numpy(np.asarray(w.is_pad, np.uint8)).cuda()
    tt = dev_i32(toks)
    with torch.cuda.stream(side):
        got = pvc.pack_tokens(meta["cu_seqlens"], tt, pt, stream=side)
        # through the C ABI into a count word that starts dirty
        dirty = torch.full((1,), 12345, dtype=torch.int64, device="cuda")
        st = pvc._lib.pvc_pack_tokens(pvc._ptr(meta["cu_seqlens"]), pvc._ptr(pt), pvc._ptr(tt), w.nseg,
                                      w.total_tokens, -100, None, None, None, None, pvc._ptr(dirty),
                                      pvc._ptr(got["dev_error"]), pvc._stream(side))
        assert st == 0
    torch.cuda.synchronize()
    assert int(dirty.item()) == ref["num_targets"]
    say(f"  pack_tokens {name}: T={w.total_tokens} nseg={w.nseg}")
    assert int(meta["dev_error"].item()) == 0 and int(got["dev_error"].item()) == 0
    assert (meta["cu_seqlens"].cpu().numpy() == ref["cu_seqlens"]).all()
    assert int(meta["max_seqlen"].item()) == ref["max_seqlen"]
    for key in ("segment_ids", "position_ids", "shifted_labels", "loss_mask"):
        assert (got[key].cpu().numpy() == ref[key]).all(), key
    assert int(got["num_targets"].item()) == ref["num_targets"]


def test_pack_tokens_malformed_cu(pvc):
    """A cu that ends short of T: the tokens past it get segment -1, position 0,
    an ignored label, and PVC_DEV_TOTAL."""
    cu = dev_i32([0, 3, 5])
    toks = dev_i32(np.arange(7) + 10)
    got = pvc.pack_tokens(cu, toks)
    torch.cuda.synchronize()
    assert int(got["dev_error"].item()) & 4
    seg = got["segment_ids"].cpu().numpy()
    assert seg.tolist() == [0, 0, 0, 1, 1, -1, -1]
    assert got["shifted_labels"].cpu().numpy().tolist() == [11, 12, -100, 14, -100, -100, -100]
    assert int(got["num_targets"].item()) == 3


@pytest.mark.parametrize("lengths", [[1], [1] * 3000, [5000], [1, 2047, 1, 1, 3000, 7]])
def test_edge_lengths(pvc, lengths):
    T = sum(lengths)
    toks = np.random.default_rng(T).integers(3, 32000, T).astype(np.int32)
    say(f"  pack_build edge nseg={len(lengths)} T={T}")
    got = _run_pack(pvc, lengths, toks, None)
    _compare(got, P.pack_build(lengths, toks))


def test_without_tokens(pvc):
    got = _run_pack(pvc, [3, 2, 4], None, None, T=9)
    assert got["cu_seqlens"].tolist() == [0, 3, 5, 9]
    assert "shifted_labels" not in got


@pytest.mark.parametrize("lengths,T,bits", [
    ([3, 0, 4], 7, P.ERR_LENGTH),
    ([3, -2, 4], 5, P.ERR_LENGTH),
    ([3, 2, 4], 10, P.ERR_TOTAL),
    ([3, 2, 4], 8, P.ERR_TOTAL),
])
def test_error_bits(pvc, lengths, T, bits):
    toks = np.full(T, 7, np.int32)
    say(f"  pack_build error case {lengths} T={T}")
    got = _run_pack(pvc, lengths, toks, None)
    assert got["dev_error"][0] & bits
    if bits != P.ERR_TOTAL:           # the oracle takes T from the lengths themselves
        assert P.pack_build(lengths, toks[:sum(lengths)])["error"] & bits


def test_validate_bits(pvc, golden):
    bad = golden("packing_examples.json")["bad_prefix"]
    cases = [
        ([0, 3, 5, 9], 9, 4, None),
        ([1, 3, 5, 9], 9, 4, None),
        ([0, 3, 3, 9], 9, 6, None),
        ([0, 5, 3, 9], 9, 6, None),
        ([0, 3, 5, 8], 9, 4, None),
        ([0, 3, 5, 9], 9, 3, None),
        (bad["cu_seqlens"], 9, 4, None),
        (bad["cu_seqlens"], 9, 4, bad["lengths"]),
    ]
    for cu, T, mx, lens in cases:
        err = pvc.validate_cu_seqlens(dev_i32(cu), T, mx, None if lens is None else dev_i32(lens))
        torch.cuda.synchronize()
        assert int(err.item()) == P.validate_cu(cu, T, mx, lens), (cu, T, mx, lens)


@pytest.mark.parametrize("name", ["sft", "short"])
def test_pack_tokens_unaligned_outputs(pvc, name):
    """Outputs that do not start on a 16-byte boundary take the per-token
    kernel's element-at-a-time path (the vector path needs 16-byte aligned
    token ids and int32 outputs, a 4-byte aligned mask): same bits."""
    import ctypes
    w = make_workload(name, scale="small")
    T = w.total_tokens
    toks = token_ids(w)
    ref = P.pack_build(w.lengths, toks, w.is_pad)
    cu = dev_i32(ref["cu_seqlens"])
    pt = torch.from_numpy(np.asarray(w.is_pad, np.uint8)).cuda()
    tbuf = torch.zeros(T + 1, dtype=torch.int32, device="cuda")
    tbuf[1:] = dev_i32(toks)
    bufs = [torch.full((T + 1,), 77, dtype=torch.int32, device="cuda") for _ in range(3)]
    mbuf = torch.full((T + 1,), 9, dtype=torch.uint8, device="cuda")
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    off = lambda t, n: ctypes.c_void_p(t.data_ptr() + n)          # noqa: E731
    say(f"  pack_tokens unaligned {name}: T={T}")
    st = pvc._lib.pvc_pack_tokens(pvc._ptr(cu), pvc._ptr(pt), off(tbuf, 4), w.nseg, T, -100, off(bufs[0], 4),
                                  off(bufs[1], 4), off(bufs[2], 4), off(mbuf, 1), pvc._ptr(count), pvc._ptr(err),
                                  pvc._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = [b.cpu().numpy()[1:] for b in bufs]
    assert (got[0] == ref["segment_ids"]).all()
    assert (got[1] == ref["position_ids"]).all()
    assert (got[2] == ref["shifted_labels"]).all()
    assert (mbuf.cpu().numpy()[1:] == ref["loss_mask"]).all()
    assert int(count.item()) == ref["num_targets"]
