"""The allocation-free forward (pvc_varlen_attn_fwd_noalloc) against the
forward it varies (pvc_varlen_attn_fwd with a caller workspace), both called
through the C ABI: two calls in a row on the library's static plan memory,
the second with a smaller input, must each give the existing entry point's
outputs bit for bit (same plan, same kernels, deterministic).  Also: a call
beyond the static limit is refused with PVC_ERR_SCRATCH_LIMIT, and a call
with a malformed cu_seqlens after a good one sets the error bits and writes
nothing (the stale plan from the previous call is not used)."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import host_bits, say
from oracle import pack as P
from workloads import make_workload

pytestmark = pytest.mark.gpu

ERR_SCRATCH_LIMIT = 6


@pytest.fixture(scope="module")
def pvc():
    import packed_varlen_causal_amd as m
    assert torch.cuda.is_available()
    return m


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _case(name, heads, d, seed):
    w = make_workload(name, scale="small" if name != "sft" else "full")
    cu = P.pack_build(w.lengths)["cu_seqlens"].astype(np.int32)
    T = int(cu[-1])
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q, k, v = (torch.randn((T, heads, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    return q, k, v, torch.from_numpy(cu).cuda(), int(np.diff(cu).max())


def _existing(pvc, q, k, v, cu, mx, code):
    T, H, D = q.shape
    ws_bytes = pvc._lib.pvc_varlen_attn_fwd_workspace_size(T, cu.numel() - 1, mx, H, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H, D), dtype=torch.float32 if code == 1 else torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = pvc._lib.pvc_varlen_attn_fwd(_vp(q), _vp(k), _vp(v), _vp(out), _vp(lse), _vp(cu), cu.numel() - 1, T, mx,
                                      H, D, 1, code, _vp(ws), ws_bytes, _vp(err), _stream())
    assert st == 0
    return out, lse, err


def _noalloc(pvc, q, k, v, cu, mx, code):
    T, H, D = q.shape
    out = torch.full((T, H, D), 3.0, dtype=torch.float32 if code == 1 else torch.bfloat16, device="cuda")
    lse = torch.full((H, T), 3.0, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = pvc._lib.pvc_varlen_attn_fwd_noalloc(_vp(q), _vp(k), _vp(v), _vp(out), _vp(lse), _vp(cu), cu.numel() - 1,
                                              T, mx, H, D, 1, code, _vp(err), _stream())
    return st, out, lse, err


def test_two_calls_in_a_row_match_the_workspace_entry_point(pvc):
    cases = [("sft", 8, 128, 1, 0), ("pretrain", 2, 64, 2, 1)]   # the second smaller, fp32 output
    for name, H, d, seed, code in cases:
        q, k, v, cu, mx = _case(name, H, d, seed)
        say(f"  noalloc {name}: T={q.shape[0]} nseg={cu.numel() - 1} H={H} d={d} out={'f32' if code else 'bf16'}")
        st, out, lse, err = _noalloc(pvc, q, k, v, cu, mx, code)
        assert st == 0
        ref, ref_lse, ref_err = _existing(pvc, q, k, v, cu, mx, code)
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and int(ref_err.item()) == 0
        if code == 1:
            assert torch.equal(out, ref)
        else:
            assert (host_bits(out) == host_bits(ref)).all()
        assert torch.equal(lse, ref_lse)


def test_bad_cu_after_a_good_call_writes_nothing(pvc):
    q, k, v, cu, mx = _case("pretrain", 2, 64, 3)
    st, _, _, err = _noalloc(pvc, q, k, v, cu, mx, 0)
    assert st == 0
    bad = cu.clone()
    bad[1] = bad[2]                                   # a zero-length segment
    st, out, lse, err = _noalloc(pvc, q, k, v, bad, mx, 0)
    torch.cuda.synchronize()
    assert st == 0
    assert int(err.item()) & 2                        # PVC_DEV_NOT_INCREASING
    assert (out.float() == 3.0).all() and (lse == 3.0).all()


def test_beyond_the_static_limit_is_refused(pvc):
    limit = int(pvc._lib.pvc_noalloc_max_tokens())
    assert limit == 1 << 20
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, limit + 1], dtype=torch.int32, device="cuda")
    st = pvc._lib.pvc_varlen_attn_fwd_noalloc(_vp(x), _vp(x), _vp(x), _vp(x), None, _vp(cu), 1, limit + 1,
                                              limit + 1, 1, 64, 1, 0, None, _stream())
    assert st == ERR_SCRATCH_LIMIT
