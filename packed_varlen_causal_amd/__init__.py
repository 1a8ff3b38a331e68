"""Packed variable-length causal attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libpvc.so`` (declared in
``include/pvc.h``).  This module only marshals arguments: it checks tensor
shapes and dtypes, allocates outputs with PyTorch and passes device pointers
and the current HIP stream to the library.  Every step of the computation runs
in the library's HIP kernels; there is no fallback path, and importing the
package fails if the library has not been built.

Entry points (same names as the C ABI without the ``pvc_`` prefix):
  pack_build            cu_seqlens, segment ids, positions, shifted labels,
                        loss mask, int64 target count, max_seqlen
  pack_tokens           the per-token part of pack_build on a given cu_seqlens
  validate_cu_seqlens   device-side check of a caller cu_seqlens
  rope_thd_apply        per-segment rotary embedding on q and k
  attn_plan             tile plan for one cu_seqlens (reusable across layers)
  varlen_attn_fwd       block-diagonal (causal) attention over THD q/k/v
  varlen_attn_bwd       its gradients dq, dk, dv on the same plan
  padded_attn_fwd_sbhd  the same kernel on a padded SBHD buffer (measurement)
  attn_plan_qk, varlen_attn_fwd_qk  prefill: separate query / key boundaries
                        (bottom-right causal) and grouped key / value heads
  packed_ce_loss        cross-entropy over the packed rows: loss sum, int64
                        target count, optional per-row / per-segment values and
                        the fused gradient
"""

from __future__ import annotations

import ctypes
import functools
import os

import torch

__all__ = [
    "PvcError", "DEV_ERROR_BITS", "lib_path", "pack_build", "pack_tokens", "validate_cu_seqlens",
    "rope_thd_apply", "AttnPlan", "attn_plan", "varlen_attn_fwd", "varlen_attn_bwd",
    "padded_attn_fwd_sbhd", "error_names", "attn_workspace_size", "attn_bwd_scratch_size",
    "packed_ce_loss", "ce_workspace_size", "AttnPlanQK", "attn_plan_qk", "varlen_attn_fwd_qk",
    "varlen_attn_fwd_noalloc", "noalloc_max_tokens",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libpvc.so")

OK, ERR_NULL, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = range(7)
OUT_BF16, OUT_F32, OUT_F16, OUT_F16_F32 = 0, 1, 2, 3
DEV_ERROR_BITS = {
    1: "CU0", 2: "NOT_INCREASING", 4: "TOTAL", 8: "MAXSEQ", 16: "LENGTH",
    32: "MISMATCH", 64: "RANGE", 128: "PLAN", 256: "LABEL", 512: "PADDED",
}


class PvcError(RuntimeError):
    """A libpvc entry point returned a non-zero status, or device data was invalid."""


def _load() -> ctypes.CDLL:
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build the HIP library first "
            "(python -m packed_varlen_causal_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(lib_path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "pvc_status_string": ([I32], ctypes.c_char_p),
        "pvc_version": ([], ctypes.c_char_p),
        "pvc_pack_build_workspace_size": ([I32, I64], SZ),
        "pvc_pack_build": ([P, P, P, I32, I64, I32, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "pvc_pack_tokens": ([P, P, P, I32, I64, I32, P, P, P, P, P, P, P], I32),
        "pvc_validate_cu_seqlens": ([P, I32, I64, I32, P, P, P], I32),
        "pvc_rope_thd_apply": ([P, P, P, P, I64, I32, I32, P, I32, F32, P, P], I32),
        "pvc_rope_thd_apply_interleaved": ([P, P, P, P, I64, I32, I32, P, I32, F32, P, P], I32),
        "pvc_rope_thd_apply_ex": ([P, P, P, P, I64, I32, I32, P, I32, F32, I32, P, P], I32),
        "pvc_attn_workspace_size": ([I64, I32], SZ),
        "pvc_attn_plan": ([P, I32, I64, I32, I32, P, SZ, P, P], I32),
        "pvc_attn_plan_padded": ([P, P, I32, I64, I32, I32, P, SZ, P, P], I32),
        "pvc_attn_plan_qk": ([P, P, I32, I64, I64, I32, I32, I32, P, SZ, P, P], I32),
        "pvc_varlen_attn_fwd_qk_planned": ([P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, P, SZ, P, P], I32),
        "pvc_varlen_attn_fwd_planned": ([P, P, P, P, P, I64, I32, I32, I32, I32, P, SZ, P, P], I32),
        "pvc_varlen_attn_fwd": ([P, P, P, P, P, P, I32, I64, I32, I32, I32, I32, I32, P, SZ, P, P], I32),
        "pvc_varlen_attn_fwd_workspace_size": ([I64, I32, I32, I32, I32], SZ),
        "pvc_noalloc_max_tokens": ([], I64),
        "pvc_varlen_attn_fwd_noalloc": ([P, P, P, P, P, P, I32, I64, I32, I32, I32, I32, I32, P, P], I32),
        "pvc_padded_attn_fwd_sbhd": ([P, P, P, P, P, I32, I32, I32, I32, I32, I32, P], I32),
        "pvc_attn_bwd_scratch_size": ([I64, I32], SZ),
        "pvc_varlen_attn_bwd_planned": ([P, P, P, P, P, P, P, P, P, I64, I32, I32, I32, I32, P, SZ, P, SZ,
                                         P, P], I32),
        "pvc_ce_workspace_size": ([I64], SZ),
        "pvc_packed_ce_loss": ([P, I32, I64, P, I64, I32, I32, P, I32, P, P, P, P, P, P, I32, I64, F32, P, SZ,
                                P, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def version() -> str:
    return _lib.pvc_version().decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise PvcError(f"{what}: {_lib.pvc_status_string(status).decode()} (status {status})")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run ``fn`` with ``stream`` (when given) as torch's current stream, so
    that every tensor it allocates (outputs, plan workspaces, scratch, error
    words) belongs to the stream the library enqueues on.  Temporaries freed
    on return then go back to that stream's pool and are not handed to other
    work while the enqueued kernels still read them."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _io_code(in_dtype: torch.dtype, out_dtype: torch.dtype) -> int:
    """The library's out_dtype code for 16-bit inputs of in_dtype."""
    if in_dtype == torch.bfloat16 and out_dtype in (torch.bfloat16, torch.float32):
        return OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if in_dtype == torch.float16 and out_dtype in (torch.float16, torch.float32):
        return OUT_F16_F32 if out_dtype == torch.float32 else OUT_F16
    raise TypeError(f"out_dtype must be the inputs' dtype or torch.float32 (inputs {in_dtype}, out {out_dtype})")


def _require16(ts, names) -> torch.dtype:
    """bf16 or fp16 tensors, all of one dtype; returns it."""
    dt = ts[0].dtype
    if dt not in (torch.bfloat16, torch.float16):
        raise TypeError(f"{names[0]} must be bf16 or fp16")
    for t, n in zip(ts, names):
        _require(t, n, dt, 3)
    return dt


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def error_names(bits: int) -> list[str]:
    return [n for b, n in DEV_ERROR_BITS.items() if bits & b]


def _raise_dev(err: torch.Tensor, what: str) -> None:
    bits = int(err.item())
    if bits:
        raise PvcError(f"{what}: invalid device data ({', '.join(error_names(bits))})")


def _new_error_word(device) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


# ------------------------------------------------------------------ packing

@_on_stream
def pack_build(lengths: torch.Tensor, tokens: torch.Tensor | None = None,
               is_pad: torch.Tensor | None = None, ignore_index: int = -100,
               total_tokens: int | None = None, dev_error: torch.Tensor | None = None,
               check: bool = False, stream=None, per_token: bool = True) -> dict:
    """Packing metadata on the GPU.

    lengths int32 [nseg] (device), tokens int32 [T] (device, optional),
    is_pad uint8 [nseg] (optional).  ``total_tokens`` defaults to tokens.numel().
    Returns a dict of device tensors.  ``check=True`` synchronizes and raises on
    device error bits.  ``per_token=False`` computes only cu_seqlens and
    max_seqlen (the per-token pass can then run apart: :func:`pack_tokens`).
    """
    _require(lengths, "lengths", torch.int32, 1)
    dev = lengths.device
    nseg = lengths.numel()
    if tokens is not None:
        _require(tokens, "tokens", torch.int32, 1)
        T = tokens.numel() if total_tokens is None else int(total_tokens)
        if tokens.numel() != T:
            raise ValueError("tokens.numel() must equal total_tokens")
    elif total_tokens is None:
        raise ValueError("total_tokens is required when tokens is not given")
    else:
        T = int(total_tokens)
    if is_pad is not None:
        _require(is_pad, "is_pad", torch.uint8, 1)
        if is_pad.numel() != nseg:
            raise ValueError("is_pad must have one flag per segment")
    err = _new_error_word(dev) if dev_error is None else dev_error
    out = {
        "cu_seqlens": torch.empty(nseg + 1, dtype=torch.int32, device=dev),
        "max_seqlen": torch.empty(1, dtype=torch.int32, device=dev),
        "dev_error": err,
    }
    if per_token:
        out["segment_ids"] = torch.empty(T, dtype=torch.int32, device=dev)
        out["position_ids"] = torch.empty(T, dtype=torch.int32, device=dev)
    if per_token and tokens is not None:
        out["shifted_labels"] = torch.empty(T, dtype=torch.int32, device=dev)
        out["loss_mask"] = torch.empty(T, dtype=torch.uint8, device=dev)
        out["num_targets"] = torch.empty(1, dtype=torch.int64, device=dev)
    ws_bytes = _lib.pvc_pack_build_workspace_size(nseg, T)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = _lib.pvc_pack_build(
        _ptr(lengths), _ptr(is_pad), _ptr(tokens), nseg, T, ignore_index, _ptr(out["cu_seqlens"]),
        _ptr(out.get("segment_ids")), _ptr(out.get("position_ids")), _ptr(out.get("shifted_labels")),
        _ptr(out.get("loss_mask")), _ptr(out.get("num_targets")), _ptr(out["max_seqlen"]),
        _ptr(err), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "pack_build")
    if check:
        _raise_dev(err, "pack_build")
    return out


@_on_stream
def pack_tokens(cu_seqlens: torch.Tensor, tokens: torch.Tensor | None = None, is_pad: torch.Tensor | None = None,
                ignore_index: int = -100, total_tokens: int | None = None, dev_error: torch.Tensor | None = None,
                check: bool = False, stream=None) -> dict:
    """The per-token pass of :func:`pack_build` on an existing cu_seqlens
    (int32 [nseg + 1], device): segment_ids, position_ids and, with tokens,
    shifted_labels, loss_mask and num_targets."""
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    dev = cu_seqlens.device
    nseg = cu_seqlens.numel() - 1
    if tokens is not None:
        _require(tokens, "tokens", torch.int32, 1)
        T = tokens.numel() if total_tokens is None else int(total_tokens)
        if tokens.numel() != T:
            raise ValueError("tokens.numel() must equal total_tokens")
    elif total_tokens is None:
        raise ValueError("total_tokens is required when tokens is not given")
    else:
        T = int(total_tokens)
    if is_pad is not None:
        _require(is_pad, "is_pad", torch.uint8, 1)
        if is_pad.numel() != nseg:
            raise ValueError("is_pad must have one flag per segment")
    err = _new_error_word(dev) if dev_error is None else dev_error
    out = {
        "segment_ids": torch.empty(T, dtype=torch.int32, device=dev),
        "position_ids": torch.empty(T, dtype=torch.int32, device=dev),
        "dev_error": err,
    }
    if tokens is not None:
        out["shifted_labels"] = torch.empty(T, dtype=torch.int32, device=dev)
        out["loss_mask"] = torch.empty(T, dtype=torch.uint8, device=dev)
        out["num_targets"] = torch.empty(1, dtype=torch.int64, device=dev)
    st = _lib.pvc_pack_tokens(
        _ptr(cu_seqlens), _ptr(is_pad), _ptr(tokens), nseg, T, ignore_index, _ptr(out["segment_ids"]),
        _ptr(out["position_ids"]), _ptr(out.get("shifted_labels")), _ptr(out.get("loss_mask")),
        _ptr(out.get("num_targets")), _ptr(err), _stream(stream))
    _check(st, "pack_tokens")
    if check:
        _raise_dev(err, "pack_tokens")
    return out


@_on_stream
def validate_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int, max_seqlen: int,
                        lengths: torch.Tensor | None = None, dev_error: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """OR the contract violations of cu_seqlens into an int32 error word (returned)."""
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if lengths is not None:
        _require(lengths, "lengths", torch.int32, 1)
    err = _new_error_word(cu_seqlens.device) if dev_error is None else dev_error
    st = _lib.pvc_validate_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(total_tokens),
                                      int(max_seqlen), _ptr(lengths), _ptr(err), _stream(stream))
    _check(st, "validate_cu_seqlens")
    return err


# --------------------------------------------------------------------- RoPE

@_on_stream
def rope_thd_apply(q: torch.Tensor, k: torch.Tensor | None, cu_seqlens: torch.Tensor,
                   base: float = 10000.0, q_out: torch.Tensor | None = None,
                   k_out: torch.Tensor | None = None, dev_error: torch.Tensor | None = None,
                   stream=None, interleaved: bool = False):
    """Per-segment RoPE on bf16 or fp16 [T, H, d] q (and k).  In place unless
    outputs are given.  Rotate-half pairing, or (x_2j, x_2j+1) pairs with
    ``interleaved=True``."""
    dt = _require16((q,), ("q",))
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, H, D = q.shape
    q_out = q if q_out is None else q_out
    _require(q_out, "q_out", dt, 3)
    if q_out.shape != q.shape:
        raise ValueError("q_out must match q")
    if k is not None:
        _require(k, "k", dt, 3)
        if k.shape != q.shape:
            raise ValueError("k must have q's shape")
        k_out = k if k_out is None else k_out
        _require(k_out, "k_out", dt, 3)
        if k_out.shape != q.shape:
            raise ValueError("k_out must match k")
    err = dev_error
    flags = (1 if interleaved else 0) | (2 if dt == torch.float16 else 0)
    st = _lib.pvc_rope_thd_apply_ex(_ptr(q), _ptr(q_out), _ptr(k), _ptr(k_out if k is not None else None),
                                    T, H, D, _ptr(cu_seqlens), cu_seqlens.numel() - 1, float(base), flags,
                                    _ptr(err), _stream(stream))
    _check(st, "rope_thd_apply")
    return q_out, (k_out if k is not None else None)


# ---------------------------------------------------------------- attention

def attn_workspace_size(total_tokens: int, nseg: int) -> int:
    return int(_lib.pvc_attn_workspace_size(int(total_tokens), int(nseg)))


class AttnPlan:
    """Device tile plan for one cu_seqlens; reusable by every layer and head.

    With ``cu_seqlens_padded`` the buffers hold padded storage: segment r's
    tokens at rows [cu_seqlens_padded[r], + L_r) and ``total_tokens`` is the
    number of storage rows (see pvc_attn_plan_padded)."""

    @_on_stream
    def __init__(self, cu_seqlens: torch.Tensor, total_tokens: int, max_seqlen: int,
                 causal: bool = True, dev_error: torch.Tensor | None = None, stream=None,
                 workspace: torch.Tensor | None = None, cu_seqlens_padded: torch.Tensor | None = None):
        _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
        self.total_tokens = int(total_tokens)
        self.nseg = cu_seqlens.numel() - 1
        self.causal = bool(causal)
        self.cu_seqlens = cu_seqlens
        self.dev_error = _new_error_word(cu_seqlens.device) if dev_error is None else dev_error
        self.ws_bytes = attn_workspace_size(self.total_tokens, self.nseg)
        if workspace is None:
            workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=cu_seqlens.device)
        elif workspace.numel() < self.ws_bytes:
            raise ValueError("workspace too small")
        self.workspace = workspace
        self.cu_seqlens_padded = cu_seqlens_padded
        if cu_seqlens_padded is None:
            st = _lib.pvc_attn_plan(_ptr(cu_seqlens), self.nseg, self.total_tokens, int(max_seqlen),
                                    int(self.causal), _ptr(workspace), self.ws_bytes, _ptr(self.dev_error),
                                    _stream(stream))
        else:
            _require(cu_seqlens_padded, "cu_seqlens_padded", torch.int32, 1)
            if cu_seqlens_padded.numel() != cu_seqlens.numel():
                raise ValueError("cu_seqlens_padded must have one entry per cu_seqlens entry")
            st = _lib.pvc_attn_plan_padded(_ptr(cu_seqlens), _ptr(cu_seqlens_padded), self.nseg,
                                           self.total_tokens, int(max_seqlen), int(self.causal), _ptr(workspace),
                                           self.ws_bytes, _ptr(self.dev_error), _stream(stream))
        _check(st, "attn_plan")


def attn_plan(cu_seqlens, total_tokens, max_seqlen, causal=True, **kw) -> AttnPlan:
    return AttnPlan(cu_seqlens, total_tokens, max_seqlen, causal, **kw)


class AttnPlanQK:
    """Plan for separate query / key boundaries (pvc_attn_plan_qk)."""

    @_on_stream
    def __init__(self, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, total_q: int, total_k: int,
                 max_seqlen_q: int, max_seqlen_k: int, causal: bool = True,
                 dev_error: torch.Tensor | None = None, stream=None, workspace: torch.Tensor | None = None):
        _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
        _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k must have one entry per request + 1")
        self.total_q, self.total_k = int(total_q), int(total_k)
        self.nseg = cu_seqlens_q.numel() - 1
        self.causal = bool(causal)
        self.dev_error = _new_error_word(cu_seqlens_q.device) if dev_error is None else dev_error
        self.ws_bytes = attn_workspace_size(self.total_q, self.nseg)
        if workspace is None:
            workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=cu_seqlens_q.device)
        elif workspace.numel() < self.ws_bytes:
            raise ValueError("workspace too small")
        self.workspace = workspace
        st = _lib.pvc_attn_plan_qk(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), self.nseg, self.total_q, self.total_k,
                                   int(max_seqlen_q), int(max_seqlen_k), int(self.causal), _ptr(workspace),
                                   self.ws_bytes, _ptr(self.dev_error), _stream(stream))
        _check(st, "attn_plan_qk")


def attn_plan_qk(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k, causal=True,
                 **kw) -> AttnPlanQK:
    return AttnPlanQK(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k, causal, **kw)


@_on_stream
def varlen_attn_fwd_qk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       cu_seqlens_q: torch.Tensor | None = None, cu_seqlens_k: torch.Tensor | None = None,
                       max_seqlen_q: int | None = None, max_seqlen_k: int | None = None, causal: bool = True,
                       return_lse: bool = False, out_dtype: torch.dtype | None = None,
                       plan: AttnPlanQK | None = None, out: torch.Tensor | None = None, check: bool = False,
                       stream=None):
    """Prefill attention: q [Tq, H, d] over k, v [Tk, Hkv, d] (bf16 or fp16, H a
    multiple of Hkv) with separate request boundaries; bottom-right causal alignment."""
    in_dt = _require16((q, k, v), ("q", "k", "v"))
    Tq, H, D = q.shape
    Tk, Hkv, Dk = k.shape
    if v.shape != k.shape or Dk != D:
        raise ValueError("k and v must share the shape [Tk, Hkv, d] with q's d")
    if H % Hkv:
        raise ValueError("the query heads must be a multiple of the key / value heads")
    out_dtype = in_dt if out_dtype is None else out_dtype
    code = _io_code(in_dt, out_dtype)
    if plan is None:
        if cu_seqlens_q is None or cu_seqlens_k is None or max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("give both cu_seqlens and max_seqlens, or a plan")
        plan = AttnPlanQK(cu_seqlens_q, cu_seqlens_k, Tq, Tk, max_seqlen_q, max_seqlen_k, causal, stream=stream)
    elif plan.total_q != Tq or plan.total_k != Tk or plan.causal != bool(causal):
        raise ValueError("plan was built for other totals / causal")
    if out is None:
        out = torch.empty((Tq, H, D), dtype=out_dtype, device=q.device)
    else:
        _require(out, "out", out_dtype, 3)
        if tuple(out.shape) != (Tq, H, D):
            raise ValueError("out must be [Tq, H, d] like q")
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device) if return_lse else None
    st = _lib.pvc_varlen_attn_fwd_qk_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), Tq, Tk, H, Hkv, D, int(bool(causal)), code,
        _ptr(plan.workspace), plan.ws_bytes,
        _ptr(plan.dev_error), _stream(stream))
    _check(st, "varlen_attn_fwd_qk")
    if check:
        _raise_dev(plan.dev_error, "varlen_attn_fwd_qk")
    return (out, lse) if return_lse else out


@_on_stream
def varlen_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens: torch.Tensor | None = None, max_seqlen: int | None = None,
                    causal: bool = True, return_lse: bool = False,
                    out_dtype: torch.dtype | None = None, plan: AttnPlan | None = None,
                    out: torch.Tensor | None = None, check: bool = False, stream=None):
    """Block-diagonal attention over THD q, k, v [T, H, d] (bf16 or fp16; d = 64 or 128).

    Either ``cu_seqlens`` + ``max_seqlen`` (a plan is built) or a ready ``plan``.
    Returns out [T, H, d] (the inputs' dtype, or fp32 with out_dtype=torch.float32)
    and, with ``return_lse``, lse fp32 [H, T].
    """
    in_dt = _require16((q, k, v), ("q", "k", "v"))
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share the shape [T, H, d]")
    T, H, D = q.shape
    out_dtype = in_dt if out_dtype is None else out_dtype
    code = _io_code(in_dt, out_dtype)
    if plan is None:
        if cu_seqlens is None or max_seqlen is None:
            raise ValueError("give cu_seqlens and max_seqlen, or a plan")
        plan = AttnPlan(cu_seqlens, T, max_seqlen, causal, stream=stream)
    elif plan.total_tokens != T or plan.causal != bool(causal):
        raise ValueError("plan was built for other total_tokens / causal")
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=q.device)
    else:
        _require(out, "out", out_dtype, 3)
        if tuple(out.shape) != (T, H, D):
            raise ValueError("out must be [T, H, d] like q")
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if return_lse else None
    st = _lib.pvc_varlen_attn_fwd_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), T, H, D, int(bool(causal)), code,
        _ptr(plan.workspace), plan.ws_bytes, _ptr(plan.dev_error), _stream(stream))
    _check(st, "varlen_attn_fwd")
    if check:
        _raise_dev(plan.dev_error, "varlen_attn_fwd")
    return (out, lse) if return_lse else out


def noalloc_max_tokens() -> int:
    return int(_lib.pvc_noalloc_max_tokens())


@_on_stream
def varlen_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                            max_seqlen: int, causal: bool = True, out: torch.Tensor | None = None,
                            lse: torch.Tensor | None = None, dev_error: torch.Tensor | None = None,
                            stream=None):
    """varlen_attn_fwd through pvc_varlen_attn_fwd_noalloc: the plan lives in
    the library's own static device memory, so the C call allocates nothing.
    Pass ``out`` (and ``lse`` [H, T] fp32, ``dev_error``) to allocate nothing
    here either; a missing ``out`` is allocated in the inputs' dtype."""
    in_dt = _require16((q, k, v), ("q", "k", "v"))
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share the shape [T, H, d]")
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, H, D = q.shape
    if out is None:
        out = torch.empty((T, H, D), dtype=in_dt, device=q.device)
    elif out.dtype not in (in_dt, torch.float32):
        raise TypeError("out must be the inputs' dtype or torch.float32")
    _require(out, "out", out.dtype, 3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must be [T, H, d] like q")
    if lse is not None:
        _require(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (H, T):
            raise ValueError("lse must be [H, T]")
    code = _io_code(in_dt, out.dtype)
    st = _lib.pvc_varlen_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), cu_seqlens.numel() - 1, T,
        int(max_seqlen), H, D, int(bool(causal)), code, _ptr(dev_error), _stream(stream))
    _check(st, "varlen_attn_fwd_noalloc")
    return out


def attn_bwd_scratch_size(total_tokens: int, heads: int) -> int:
    return int(_lib.pvc_attn_bwd_scratch_size(total_tokens, heads))


@_on_stream
def varlen_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                    dout: torch.Tensor, lse: torch.Tensor, plan: AttnPlan, causal: bool = True,
                    grad_dtype: torch.dtype | None = None, grads=None, scratch: torch.Tensor | None = None,
                    check: bool = False, stream=None):
    """Gradients (dq, dk, dv) of varlen_attn_fwd for an upstream gradient ``dout``.

    q, k, v, out, dout [T, H, d], all bf16 or all fp16; lse fp32 [H, T] from
    the forward (return_lse=True); ``plan`` the forward's plan.  Gradients are
    in the inputs' dtype (the default), or fp32 with grad_dtype=torch.float32;
    ``grads`` may pass three output tensors.
    """
    in_dt = _require16((q, k, v, out, dout), ("q", "k", "v", "out", "dout"))
    if any(t.shape != q.shape for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out and dout must share the shape [T, H, d]")
    T, H, D = q.shape
    _require(lse, "lse", torch.float32, 2)
    if tuple(lse.shape) != (H, T):
        raise ValueError("lse must be [H, T]")
    grad_dtype = in_dt if grad_dtype is None else grad_dtype
    code = _io_code(in_dt, grad_dtype)
    if plan.total_tokens != T or plan.causal != bool(causal):
        raise ValueError("plan was built for other total_tokens / causal")
    if grads is None:
        grads = tuple(torch.empty((T, H, D), dtype=grad_dtype, device=q.device) for _ in range(3))
    else:
        if len(grads) != 3:
            raise ValueError("grads must be three tensors (dq, dk, dv)")
        for name, t in zip(("dq", "dk", "dv"), grads):
            _require(t, name, grad_dtype, 3)
            if tuple(t.shape) != (T, H, D):
                raise ValueError(f"{name} must be [T, H, d] like q")
    nb = attn_bwd_scratch_size(T, H)
    if scratch is None:
        scratch = torch.empty(nb, dtype=torch.uint8, device=q.device)
    else:
        _require(scratch, "scratch", torch.uint8, 1)
        if scratch.numel() < nb:
            raise ValueError(f"scratch must hold {nb} bytes (attn_bwd_scratch_size)")
    dq, dk, dv = grads
    st = _lib.pvc_varlen_attn_bwd_planned(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), T, H, D,
        int(bool(causal)), code, _ptr(plan.workspace),
        plan.ws_bytes, _ptr(scratch), scratch.numel(), _ptr(plan.dev_error), _stream(stream))
    _check(st, "varlen_attn_bwd")
    if check:
        _raise_dev(plan.dev_error, "varlen_attn_bwd")
    return dq, dk, dv


@_on_stream
def padded_attn_fwd_sbhd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqlens: torch.Tensor,
                         causal: bool = True, out_dtype: torch.dtype = torch.bfloat16,
                         out: torch.Tensor | None = None, stream=None):
    """The attention kernel on a padded SBHD bf16 buffer [L, B, H, d] (measurement layout)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, 4)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share the shape [L, B, H, d]")
    _require(seqlens, "seqlens", torch.int32, 1)
    L, B, H, D = q.shape
    if seqlens.numel() != B:
        raise ValueError("one length per sample")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    else:
        _require(out, "out", out_dtype, 4)
        if out.shape != q.shape:
            raise ValueError("out must be [L, B, H, d] like q")
    st = _lib.pvc_padded_attn_fwd_sbhd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(seqlens), B, L, H, D,
                                       int(bool(causal)),
                                       OUT_F32 if out_dtype == torch.float32 else OUT_BF16, _stream(stream))
    _check(st, "padded_attn_fwd_sbhd")
    return out


def ce_workspace_size(total_tokens: int) -> int:
    return int(_lib.pvc_ce_workspace_size(total_tokens))


@_on_stream
def packed_ce_loss(logits: torch.Tensor, labels: torch.Tensor, cu_seqlens: torch.Tensor | None = None,
                   ignore_index: int = -100, row_loss: bool = False, segments: bool = False,
                   grad: torch.Tensor | str | None = None, grad_dtype: torch.dtype | None = None,
                   grad_scale: float = 1.0, workspace: torch.Tensor | None = None,
                   dev_error: torch.Tensor | None = None, check: bool = False, stream=None) -> dict:
    """Cross-entropy over packed rows (see pvc_packed_ce_loss in include/pvc.h).

    logits [T, V] bf16, fp16 or fp32 (rows may be strided: stride(1) must be 1);
    labels [T] int32, the pre-shifted labels of pack_build.  Returns a dict of
    device tensors: loss_sum (fp64 [1]), target_count (int64 [1]), and on
    request row_loss (fp32 [T]), seg_loss / seg_count ([nseg], needs
    cu_seqlens) and grad.  ``grad`` is "new" (a fresh tensor of grad_dtype,
    default the logits' dtype), "inplace" (written over the logits) or a
    caller tensor of the logits' shape.
    """
    codes = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32, torch.float16: OUT_F16}
    if logits.dtype not in codes:
        raise TypeError("logits must be bf16, fp16 or fp32")
    if logits.device.type != "cuda" or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D GPU tensor with unit stride along the vocabulary")
    T, V = logits.shape
    _require(labels, "labels", torch.int32, 1)
    if labels.numel() != T:
        raise ValueError("one label per row")
    dev = logits.device
    dt = codes[logits.dtype]
    nseg = 0
    if cu_seqlens is not None:
        _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
        nseg = cu_seqlens.numel() - 1
    elif segments:
        raise ValueError("segments=True needs cu_seqlens")
    out = {"loss_sum": torch.empty(1, dtype=torch.float64, device=dev),
           "target_count": torch.empty(1, dtype=torch.int64, device=dev)}
    if row_loss:
        out["row_loss"] = torch.empty(T, dtype=torch.float32, device=dev)
    if segments:
        out["seg_loss"] = torch.empty(nseg, dtype=torch.float64, device=dev)
        out["seg_count"] = torch.empty(nseg, dtype=torch.int64, device=dev)
    g = None
    if isinstance(grad, str):
        if grad == "inplace":
            if grad_dtype not in (None, logits.dtype):
                raise ValueError("an in-place gradient has the logits' dtype")
            g = logits
        elif grad == "new":
            g = torch.empty((T, V), dtype=grad_dtype or logits.dtype, device=dev)
        else:
            raise ValueError('grad must be None, "new", "inplace" or a tensor')
    elif grad is not None:
        g = grad
        if g.dtype not in codes or g.dim() != 2 or tuple(g.shape) != (T, V) \
                or g.stride(1) != 1 or g.device != dev:
            raise ValueError("grad must be a [T, V] bf16 / fp16 / fp32 GPU tensor with unit vocabulary stride")
    if g is not None:
        out["grad"] = g
    nb = ce_workspace_size(T)
    if workspace is None:
        workspace = torch.empty(nb, dtype=torch.uint8, device=dev)
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        if workspace.numel() < nb:
            raise ValueError(f"workspace must hold {nb} bytes (ce_workspace_size)")
    if dev_error is None:
        dev_error = torch.zeros(1, dtype=torch.int32, device=dev)
    gdt = 0 if g is None else codes[g.dtype]
    st = _lib.pvc_packed_ce_loss(
        _ptr(logits), dt, logits.stride(0), _ptr(labels), T, V, ignore_index, _ptr(cu_seqlens), nseg,
        _ptr(out["loss_sum"]), _ptr(out["target_count"]), _ptr(out.get("row_loss")), _ptr(out.get("seg_loss")),
        _ptr(out.get("seg_count")), _ptr(g), gdt, 0 if g is None else g.stride(0), float(grad_scale),
        _ptr(workspace), workspace.numel(), _ptr(dev_error), _stream(stream))
    _check(st, "packed_ce_loss")
    out["dev_error"] = dev_error
    if check:
        _raise_dev(dev_error, "packed_ce_loss")
    return out
