"""The C ABI library loads and exports every symbol include/pvc.h declares, and
its host-side argument checks reject bad calls before any GPU work (CPU only:
every call here returns before a HIP runtime call)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pvc.h")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pvc_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    path = os.path.join(ROOT, "packed_varlen_causal_amd", "libpvc.so")
    if not os.path.exists(path):
        # build.py by path: importing the package would try to load the library
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "pvc_build", os.path.join(ROOT, "packed_varlen_causal_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return ctypes.CDLL(path)


def test_header_declares_the_hot_path():
    names = declared_functions()
    for must in ("pvc_pack_build", "pvc_validate_cu_seqlens", "pvc_rope_thd_apply", "pvc_attn_plan",
                 "pvc_varlen_attn_fwd", "pvc_varlen_attn_fwd_planned", "pvc_padded_attn_fwd_sbhd",
                 "pvc_attn_workspace_size", "pvc_pack_build_workspace_size", "pvc_status_string",
                 "pvc_varlen_attn_bwd_planned", "pvc_attn_bwd_scratch_size", "pvc_packed_ce_loss",
                 "pvc_ce_workspace_size", "pvc_attn_plan_padded", "pvc_rope_thd_apply_interleaved",
                 "pvc_attn_plan_qk", "pvc_varlen_attn_fwd_qk_planned", "pvc_rope_thd_apply_ex",
                 "pvc_pack_tokens", "pvc_varlen_attn_fwd_workspace_size"):
        assert must in names


def test_scoped_boundary_names_and_arities():
    """The entry points of the scoped boundary exist with the argument counts
    it lists (the departures in argument lists are supersets: RoPE takes
    separate in / out pointers, validation optional lengths, the padded
    baseline an output dtype and no workspace)."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", " ", f.read(), flags=re.S)
    arity = {m.group(1): len([a for a in m.group(2).split(",") if a.strip() not in ("", "void")])
             for m in re.finditer(r"\b(pvc_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S)}
    want = {"pvc_pack_build_workspace_size": 2, "pvc_pack_build": 17, "pvc_validate_cu_seqlens": 7,
            "pvc_rope_thd_apply": 12, "pvc_varlen_attn_fwd_workspace_size": 5, "pvc_varlen_attn_fwd": 17,
            "pvc_padded_attn_fwd_sbhd": 12, "pvc_status_string": 1}
    for name, n in want.items():
        assert arity.get(name) == n, (name, arity.get(name), n)


def test_every_declared_symbol_is_exported(lib):
    path = os.path.join(ROOT, "packed_varlen_causal_amd", "libpvc.so")
    dyn = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(pvc_\w+)", dyn))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_is_gfx950_code_object():
    """The library built here embeds a device code object for gfx950 only."""
    path = os.path.join(ROOT, "packed_varlen_causal_amd", "libpvc.so")
    sections = subprocess.run(["/opt/rocm/lib/llvm/bin/llvm-readelf", "-S", path],
                              capture_output=True, text=True, check=True).stdout
    assert ".hip_fatbin" in sections
    with open(path, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    assert b"gfx942" not in blob and b"gfx90a" not in blob


def test_status_strings(lib):
    lib.pvc_status_string.restype = ctypes.c_char_p
    lib.pvc_version.restype = ctypes.c_char_p
    assert lib.pvc_status_string(0) == b"ok"
    assert b"NULL" in lib.pvc_status_string(1)
    assert lib.pvc_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.pvc_version()


def test_workspace_queries(lib):
    lib.pvc_attn_workspace_size.restype = ctypes.c_size_t
    lib.pvc_attn_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.pvc_pack_build_workspace_size.restype = ctypes.c_size_t
    lib.pvc_pack_build_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64]
    small = lib.pvc_attn_workspace_size(9, 3)
    big = lib.pvc_attn_workspace_size(131072, 57)
    assert 0 < small < big
    assert big >= 131072 * 8            # per-row key ranges
    assert lib.pvc_attn_workspace_size(0, 1) == 0
    assert lib.pvc_pack_build_workspace_size(100, 9000) == 0
    assert lib.pvc_pack_build_workspace_size(100, (1 << 20) + 1) >= 4 * ((1 << 20) + 1) // 2048
    assert lib.pvc_pack_build_workspace_size(1 << 20, 1 << 22) > 0


def _vp(x):
    return ctypes.c_void_p(x)


def test_null_and_range_checks_return_before_gpu_work(lib):
    P = ctypes.c_void_p
    I32, I64, SZ, F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.pvc_pack_build.restype = I32
    lib.pvc_pack_build.argtypes = [P, P, P, I32, I64, I32, P, P, P, P, P, P, P, P, P, SZ, P]
    fake = _vp(0x100000)  # never dereferenced: every call below fails its host checks first
    # NULL lengths / cu
    assert lib.pvc_pack_build(None, None, None, 3, 9, -100, fake, None, None, None, None, None, None,
                              None, None, 0, None) == 1
    # labels requested without tokens
    assert lib.pvc_pack_build(fake, None, None, 3, 9, -100, fake, None, None, fake, None, None, None,
                              None, None, 0, None) == 1
    # nseg < 1, total out of int32 range
    assert lib.pvc_pack_build(fake, None, None, 0, 9, -100, fake, None, None, None, None, None, None,
                              None, None, 0, None) == 2
    assert lib.pvc_pack_build(fake, None, None, 3, 1 << 31, -100, fake, None, None, None, None, None,
                              None, None, None, 0, None) == 2
    # large nseg needs a workspace
    assert lib.pvc_pack_build(fake, None, None, 1 << 20, 1 << 22, -100, fake, None, None, None, None,
                              None, None, None, None, 0, None) == 4

    lib.pvc_pack_tokens.restype = I32
    lib.pvc_pack_tokens.argtypes = [P, P, P, I32, I64, I32, P, P, P, P, P, P, P]
    assert lib.pvc_pack_tokens(None, None, None, 3, 9, -100, fake, None, None, None, None, None, None) == 1
    assert lib.pvc_pack_tokens(fake, None, None, 3, 9, -100, None, None, fake, None, None, None, None) == 1
    assert lib.pvc_pack_tokens(fake, None, None, 0, 9, -100, fake, None, None, None, None, None, None) == 2
    assert lib.pvc_pack_tokens(fake, None, None, 3, 0, -100, fake, None, None, None, None, None, None) == 2

    lib.pvc_rope_thd_apply.restype = I32
    lib.pvc_rope_thd_apply.argtypes = [P, P, P, P, I64, I32, I32, P, I32, F32, P, P]
    assert lib.pvc_rope_thd_apply(None, fake, None, None, 9, 2, 64, fake, 3, 1e4, None, None) == 1
    assert lib.pvc_rope_thd_apply(fake, fake, fake, None, 9, 2, 64, fake, 3, 1e4, None, None) == 1
    assert lib.pvc_rope_thd_apply(fake, fake, None, None, 9, 2, 63, fake, 3, 1e4, None, None) == 3
    assert lib.pvc_rope_thd_apply(fake, fake, None, None, 9, 2, 512, fake, 3, 1e4, None, None) == 3
    assert lib.pvc_rope_thd_apply(fake, fake, None, None, 9, 2, 64, fake, 3, -1.0, None, None) == 2
    lib.pvc_rope_thd_apply_ex.restype = I32
    lib.pvc_rope_thd_apply_ex.argtypes = [P, P, P, P, I64, I32, I32, P, I32, F32, I32, P, P]
    assert lib.pvc_rope_thd_apply_ex(fake, fake, None, None, 9, 2, 64, fake, 3, 1e4, 4, None, None) == 2
    assert lib.pvc_rope_thd_apply_ex(fake, fake, None, None, 9, 2, 63, fake, 3, 1e4, 3, None, None) == 3

    lib.pvc_attn_plan.restype = I32
    lib.pvc_attn_plan.argtypes = [P, I32, I64, I32, I32, P, SZ, P, P]
    assert lib.pvc_attn_plan(None, 3, 9, 4, 1, fake, 1 << 20, None, None) == 1
    assert lib.pvc_attn_plan(fake, 3, 9, 4, 1, fake, 16, None, None) == 4
    assert lib.pvc_attn_plan(fake, 3, 9, 0, 1, fake, 1 << 20, None, None) == 2
    lib.pvc_attn_plan_padded.restype = I32
    lib.pvc_attn_plan_padded.argtypes = [P, P, I32, I64, I32, I32, P, SZ, P, P]
    assert lib.pvc_attn_plan_padded(fake, None, 3, 12, 4, 1, fake, 1 << 20, None, None) == 1
    assert lib.pvc_attn_plan_padded(fake, fake, 0, 12, 4, 1, fake, 1 << 20, None, None) == 2
    assert lib.pvc_attn_plan_padded(fake, fake, 3, 12, 4, 1, fake, 16, None, None) == 4
    lib.pvc_attn_plan_qk.restype = I32
    lib.pvc_attn_plan_qk.argtypes = [P, P, I32, I64, I64, I32, I32, I32, P, SZ, P, P]
    assert lib.pvc_attn_plan_qk(fake, None, 2, 9, 20, 8, 16, 1, fake, 1 << 20, None, None) == 1
    assert lib.pvc_attn_plan_qk(fake, fake, 2, 9, 0, 8, 16, 1, fake, 1 << 20, None, None) == 2
    lib.pvc_varlen_attn_fwd_qk_planned.restype = I32
    lib.pvc_varlen_attn_fwd_qk_planned.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, P, SZ, P, P]
    qq, kk, vv, oo = (_vp(0x10000000 * (i + 1)) for i in range(4))
    assert lib.pvc_varlen_attn_fwd_qk_planned(qq, kk, vv, oo, None, 9, 20, 6, 4, 64, 1, 0, fake, 1 << 20,
                                              None, None) == 2   # 6 heads over 4 kv heads
    assert lib.pvc_varlen_attn_fwd_qk_planned(qq, kk, vv, oo, None, 9, 20, 8, 2, 80, 1, 0, fake, 1 << 20,
                                              None, None) == 3
    assert lib.pvc_varlen_attn_fwd_qk_planned(qq, kk, vv, kk, None, 9, 20, 8, 2, 64, 1, 0, fake, 1 << 20,
                                              None, None) == 2   # out aliasing k

    lib.pvc_varlen_attn_fwd_planned.restype = I32
    lib.pvc_varlen_attn_fwd_planned.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, P, SZ, P, P]
    a, b, c, o = (_vp(0x100000 * (i + 1)) for i in range(4))
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, o, None, 9, 2, 96, 1, 0, fake, 1 << 20, None, None) == 3
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, o, None, 9, 2, 64, 1, 7, fake, 1 << 20, None, None) == 2
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, o, None, 9, 2, 64, 1, 4, fake, 1 << 20, None, None) == 2
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, None, None, 9, 2, 64, 1, 0, fake, 1 << 20, None, None) == 1
    # misaligned q
    assert lib.pvc_varlen_attn_fwd_planned(_vp(0x100002), b, c, o, None, 9, 2, 64, 1, 0, fake, 1 << 20,
                                           None, None) == 2
    # out aliasing q
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, a, None, 9, 2, 64, 1, 0, fake, 1 << 20, None, None) == 2
    # workspace too small for 9 tokens
    assert lib.pvc_varlen_attn_fwd_planned(a, b, c, o, None, 9, 2, 64, 1, 0, fake, 8, None, None) == 4
    # plan + forward: the forward's checks come before the plan is enqueued (a
    # launch here, with no GPU, would report PVC_ERR_HIP instead)
    lib.pvc_varlen_attn_fwd.restype = I32
    lib.pvc_varlen_attn_fwd.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, I32, I32, I32, P, SZ, P, P]
    assert lib.pvc_varlen_attn_fwd(_vp(0x100002), b, c, o, None, fake, 2, 9, 8, 2, 64, 1, 0, fake, 1 << 20,
                                   None, None) == 2
    assert lib.pvc_varlen_attn_fwd(a, b, c, a, None, fake, 2, 9, 8, 2, 64, 1, 0, fake, 1 << 20, None, None) == 2
    assert lib.pvc_varlen_attn_fwd(a, b, c, o, None, fake, 2, 9, 8, 2, 64, 1, 0, fake, 8, None, None) == 4

    lib.pvc_padded_attn_fwd_sbhd.restype = I32
    lib.pvc_padded_attn_fwd_sbhd.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P]
    assert lib.pvc_padded_attn_fwd_sbhd(a, b, c, o, None, 2, 4, 2, 64, 1, 0, None) == 1
    assert lib.pvc_padded_attn_fwd_sbhd(a, b, c, o, fake, 0, 4, 2, 64, 1, 0, None) == 2
    assert lib.pvc_padded_attn_fwd_sbhd(a, b, c, o, fake, 2, 4, 2, 64, 1, 5, None) == 2
    assert lib.pvc_padded_attn_fwd_sbhd(a, b, c, o, fake, 2, 4, 2, 80, 1, 0, None) == 3

    lib.pvc_attn_bwd_scratch_size.restype = SZ
    lib.pvc_attn_bwd_scratch_size.argtypes = [I64, I32]
    assert lib.pvc_attn_bwd_scratch_size(0, 2) == 0
    # two fp32 rows per head, padded to 32 tokens plus one block of 64
    assert lib.pvc_attn_bwd_scratch_size(9, 2) >= 2 * 2 * (32 + 64) * 4
    lib.pvc_varlen_attn_bwd_planned.restype = I32
    lib.pvc_varlen_attn_bwd_planned.argtypes = [P] * 9 + [I64, I32, I32, I32, I32, P, SZ, P, SZ, P, P]
    g = [_vp(0x100000 * (i + 1)) for i in range(10)]   # q k v out dout lse dq dk dv scratch
    big = 1 << 20

    def bwd(*, ptrs=None, T=9, H=2, D=64, causal=1, gd=0, ws=big, sc=big):
        p = list(g if ptrs is None else ptrs)
        return lib.pvc_varlen_attn_bwd_planned(*p[:9], T, H, D, causal, gd, fake, ws, p[9], sc, None, None)

    assert bwd(ptrs=[None] + g[1:]) == 1
    assert bwd(ptrs=g[:9] + [None]) == 1
    assert bwd(D=96) == 3
    assert bwd(gd=5) == 2
    assert bwd(gd=4) == 2                                      # not an element-type code
    assert bwd(T=0) == 2
    assert bwd(ws=8) == 4
    assert bwd(sc=8) == 4
    assert bwd(ptrs=g[:6] + [_vp(0x100008)] + g[7:]) == 2      # misaligned dq
    assert bwd(ptrs=g[:7] + [g[6]] + g[8:]) == 2               # dk aliasing dq
    assert bwd(ptrs=g[:8] + [g[0]] + g[9:]) == 2               # dv aliasing q

    lib.pvc_ce_workspace_size.restype = SZ
    lib.pvc_ce_workspace_size.argtypes = [I64]
    assert lib.pvc_ce_workspace_size(0) == 0
    assert lib.pvc_ce_workspace_size(100) >= 100 * 4       # one fp32 loss per row
    lib.pvc_packed_ce_loss.restype = I32
    lib.pvc_packed_ce_loss.argtypes = [P, I32, I64, P, I64, I32, I32, P, I32, P, P, P, P, P, P, I32, I64, F32,
                                       P, SZ, P, P]
    z, lab, ls, tc = (_vp(0x1000000 * (i + 1)) for i in range(4))

    def ce(*, logits=z, dt=0, ld=64, T=9, V=64, cu=None, nseg=0, seg=None, grad=None, gdt=0, gld=64, scale=1.0,
           ws=big, labels=lab):
        return lib.pvc_packed_ce_loss(logits, dt, ld, labels, T, V, -100, cu, nseg, ls, tc, None, seg, None, grad,
                                      gdt, gld, scale, fake, ws, None, None)

    assert ce(logits=None) == 1
    assert ce(labels=None) == 1
    assert ce(seg=_vp(0x9000000)) == 1                     # segment sums without cu_seqlens
    assert ce(T=0) == 2
    assert ce(ld=63) == 2                                  # row stride below the vocabulary
    assert ce(dt=7) == 2
    assert ce(ws=8) == 4
    assert ce(cu=fake, nseg=10) == 2                       # more segments than rows
    assert ce(grad=_vp(0x1000000 + 64)) == 2               # gradient overlapping the logits
    assert ce(grad=_vp(0x9000000), scale=float("inf")) == 2


def test_python_binding_imports_without_gpu():
    import packed_varlen_causal_amd as pvc
    assert "gfx950" in pvc.version()
    assert pvc.error_names(1 | 32) == ["CU0", "MISMATCH"]


def test_noalloc_forward_refuses_beyond_its_static_scratch_before_gpu_work(lib):
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pvc_varlen_attn_fwd_noalloc.restype = I32
    lib.pvc_varlen_attn_fwd_noalloc.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, I32, I32, I32, P, P]
    lib.pvc_noalloc_max_tokens.restype = I64
    limit = lib.pvc_noalloc_max_tokens()
    assert limit == 1 << 20
    fake = _vp(0x100000)       # never dereferenced: the calls below return before any HIP call
    assert lib.pvc_varlen_attn_fwd_noalloc(fake, fake, fake, fake, None, fake, 1, limit + 1, limit + 1, 32, 128,
                                           1, 0, None, None) == 6
    assert lib.pvc_varlen_attn_fwd_noalloc(None, fake, fake, fake, None, fake, 1, 9, 9, 2, 64, 1, 0, None,
                                           None) == 1
    assert lib.pvc_varlen_attn_fwd_noalloc(fake, fake, fake, fake, None, fake, 1, 0, 9, 2, 64, 1, 0, None,
                                           None) == 2
    lib.pvc_status_string.restype = ctypes.c_char_p
    assert b"static scratch" in lib.pvc_status_string(6)
