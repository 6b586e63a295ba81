"""Python binding of libfa.so, the gfx950 fused exact-attention library.

The functions ``fa_fwd``, ``fa_fwd_ex``, ``fa_bwd``, ``fa_bwd_workspace_size``
and ``fa_strerror`` call the C ABI of ``include/fa.h`` one-to-one (device
pointers as ints, sizes as ints, a HIP stream handle as an int).  ``forward``
and ``backward`` are thin conveniences over them for torch tensors: they check
dtype, device, shape and contiguity, allocate outputs and the workspace with
torch, and pass the current stream.  All arithmetic runs in the library's HIP
kernels; there is no other implementation here and no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_preprocess",
           "fa_bwd_main", "fa_bwd_dq", "fa_fwd_varlen", "fa_fwd_varlen_workspace_size",
           "fa_varlen_max_seqlen", "fa_fwd_splitkv", "fa_fwd_splitkv_num_splits",
           "fa_fwd_splitkv_workspace_size", "fa_bwd_varlen", "fa_bwd_varlen_workspace_size",
           "fa_fwd_fp8", "fa_fwd_fp8_workspace_size", "fa_exp2_poly_eval", "fa_bwd_noalloc", "fa_strerror",
           "forward", "backward", "backward_noalloc",
           "forward_varlen", "backward_varlen", "forward_splitkv", "forward_fp8", "FaError",
           "library_path", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
_lib = None

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_ALIGN = -3
FA_ERR_WORKSPACE = -4
FA_ERR_HIP = -5
FA_ERR_TOO_LARGE = -6
FA_ERR_SCRATCH = -7
# Fixed scratch behind fa_bwd_noalloc (FA_BWD_NOALLOC_SCRATCH_BYTES in fa.h).
BWD_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = ("fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_preprocess",
            "fa_bwd_main", "fa_bwd_dq", "fa_fwd_varlen", "fa_fwd_varlen_workspace_size",
            "fa_varlen_max_seqlen", "fa_fwd_splitkv", "fa_fwd_splitkv_num_splits",
            "fa_fwd_splitkv_workspace_size", "fa_bwd_varlen", "fa_bwd_varlen_workspace_size",
            "fa_fwd_fp8", "fa_fwd_fp8_workspace_size", "fa_exp2_poly_eval", "fa_bwd_noalloc",
            "fa_strerror")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fa_strerror(status)} ({status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libfa.so (built in-tree by ``exact_attention_98_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_attention_98_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_fwd.restype = ci
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.fa_fwd_ex.restype = ci
    lib.fa_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, sz,
                           ci, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [ci] * 6 + [cf, vp]
    lib.fa_bwd_noalloc.restype = ci
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp, sz, ci, vp]
    lib.fa_bwd_preprocess.restype = ci
    lib.fa_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, sz, ci, vp]
    lib.fa_bwd_main.restype = ci
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, sz, ci, vp]
    lib.fa_bwd_dq.restype = ci
    lib.fa_fwd_varlen_workspace_size.argtypes = [ci, ci]
    lib.fa_fwd_varlen_workspace_size.restype = sz
    lib.fa_varlen_max_seqlen.argtypes = []
    lib.fa_varlen_max_seqlen.restype = ci
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, sz,
                                  vp]
    lib.fa_fwd_varlen.restype = ci
    lib.fa_fwd_splitkv_num_splits.argtypes = [ci] * 6
    lib.fa_fwd_splitkv_num_splits.restype = ci
    lib.fa_fwd_splitkv_workspace_size.argtypes = [ci] * 7
    lib.fa_fwd_splitkv_workspace_size.restype = sz
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, vp, sz,
                                   vp]
    lib.fa_fwd_splitkv.restype = ci
    lib.fa_bwd_varlen_workspace_size.argtypes = [ci] * 7
    lib.fa_bwd_varlen_workspace_size.restype = sz
    lib.fa_bwd_varlen.argtypes = [vp] * 10 + [ci] * 7 + [cf, vp, sz, ci, vp]
    lib.fa_bwd_varlen.restype = ci
    lib.fa_fwd_fp8_workspace_size.argtypes = [ci] * 5
    lib.fa_fwd_fp8_workspace_size.restype = sz
    lib.fa_fwd_fp8.argtypes = [vp] * 5 + [ci] * 6 + [cf, vp, vp, sz, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_exp2_poly_eval.argtypes = [vp, vp, ci, vp]
    lib.fa_exp2_poly_eval.restype = ci
    lib.fa_strerror.argtypes = [ci]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ----------------------------------------------------------------- raw C ABI
def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, scale, stream) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, D, int(causal), float(scale), stream)


def fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, scale, exp_poly_quarters, stream) -> int:
    return load().fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, D, int(causal), float(scale),
                            int(exp_poly_quarters), stream)


def fa_exp2_poly_eval(x, y, n, stream) -> int:
    return load().fa_exp2_poly_eval(x, y, int(n), stream)


def fa_bwd_workspace_size(B, Hq, Hkv, N, D, deterministic) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, Hkv, N, D, int(deterministic)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, causal, scale, workspace,
           workspace_bytes, deterministic, stream) -> int:
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, int(causal),
                         float(scale), workspace, workspace_bytes, int(deterministic), stream)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, causal, scale,
                   stream) -> int:
    return load().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, int(causal),
                                 float(scale), stream)


def fa_bwd_preprocess(o, dout, lse, B, Hq, Hkv, N, D, workspace, workspace_bytes, deterministic,
                      stream) -> int:
    return load().fa_bwd_preprocess(o, dout, lse, B, Hq, Hkv, N, D, workspace, workspace_bytes,
                                     int(deterministic), stream)


def fa_bwd_main(q, k, v, dout, dk, dv, B, Hq, Hkv, N, D, causal, scale, workspace,
                workspace_bytes, deterministic, stream) -> int:
    return load().fa_bwd_main(q, k, v, dout, dk, dv, B, Hq, Hkv, N, D, int(causal), float(scale),
                              workspace, workspace_bytes, int(deterministic), stream)


def fa_bwd_dq(q, k, v, dout, dq, B, Hq, Hkv, N, D, causal, scale, workspace, workspace_bytes,
              deterministic, stream) -> int:
    return load().fa_bwd_dq(q, k, v, dout, dq, B, Hq, Hkv, N, D, int(causal), float(scale),
                            workspace, workspace_bytes, int(deterministic), stream)


def fa_fwd_varlen_workspace_size(B, total) -> int:
    return int(load().fa_fwd_varlen_workspace_size(B, total))


def fa_varlen_max_seqlen() -> int:
    return int(load().fa_varlen_max_seqlen())


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, Hq, Hkv, total, max_seqlen, D, causal, scale,
                  workspace, workspace_bytes, stream) -> int:
    return load().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, Hq, Hkv, total, max_seqlen, D,
                                int(causal), float(scale), workspace, workspace_bytes, stream)


def fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, D) -> int:
    return int(load().fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, D))


def fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, num_splits) -> int:
    return int(load().fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, causal, scale, num_splits, workspace,
                   workspace_bytes, stream) -> int:
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, int(causal),
                                 float(scale), int(num_splits), workspace, workspace_bytes,
                                 stream)


def fa_bwd_varlen_workspace_size(B, Hq, Hkv, total, max_seqlen, D, deterministic) -> int:
    return int(load().fa_bwd_varlen_workspace_size(B, Hq, Hkv, total, int(max_seqlen), D,
                                                   int(deterministic)))


def fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, B, Hq, Hkv, total, max_seqlen, D,
                  causal, scale, workspace, workspace_bytes, deterministic, stream) -> int:
    return load().fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, B, Hq, Hkv, total,
                                max_seqlen, D, int(causal), float(scale), workspace,
                                workspace_bytes, int(deterministic), stream)


def fa_fwd_fp8_workspace_size(B, Hq, Hkv, N, D) -> int:
    return int(load().fa_fwd_fp8_workspace_size(B, Hq, Hkv, N, D))


def fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, scale, signs, workspace,
               workspace_bytes, stream) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N, D, int(causal), float(scale), signs,
                             workspace, workspace_bytes, stream)


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


# ------------------------------------------------------- torch conveniences
def _check(name, t, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, causal: bool, scale: float, *, exp_poly_quarters: int | None = None,
            out=None, lse=None):
    """O (bf16) and LSE (fp32) for q [B,Hq,N,D], k/v [B,Hkv,N,D] bf16 device tensors."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    _check("q", q, torch.bfloat16, (B, Hq, N, D))
    _check("k", k, torch.bfloat16, (B, Hkv, N, D))
    _check("v", v, torch.bfloat16, (B, Hkv, N, D))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check("out", out, torch.bfloat16, (B, Hq, N, D))
    _check("lse", lse, torch.float32, (B, Hq, N))
    stream = _stream_handle(q.device)
    if exp_poly_quarters is None:
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                    Hq, Hkv, N, D, causal, scale, stream)
    else:
        rc = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, N, D, causal, scale, exp_poly_quarters, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd")
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool, scale: float, *, deterministic=False,
             workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV (bf16) for the forward's inputs/outputs and dO.

    deterministic selects the dQ mode of fa_bwd: 0 / False atomic; 1 / True
    fixed order from stored dS blocks (largest workspace); 2 fixed order,
    recomputing dS (smallest workspace).
    """
    import torch
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    for name, t, shp in (("q", q, (B, Hq, N, D)), ("k", k, (B, Hkv, N, D)),
                         ("v", v, (B, Hkv, N, D)), ("o", o, (B, Hq, N, D)),
                         ("dout", dout, (B, Hq, N, D))):
        _check(name, t, torch.bfloat16, shp)
    _check("lse", lse, torch.float32, (B, Hq, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = fa_bwd_workspace_size(B, Hq, Hkv, N, D, deterministic)
    if ws_bytes == 0:
        raise FaError(FA_ERR_INVALID, "fa_bwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if workspace.numel() < ws_bytes:
        raise FaError(FA_ERR_WORKSPACE, "fa_bwd")
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, D,
                causal, scale, workspace.data_ptr(), workspace.numel(), deterministic,
                _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, dout, causal: bool, scale: float, *, dq=None, dk=None,
                     dv=None):
    """dQ, dK, dV (bf16) through fa_bwd_noalloc: fixed-order dQ recomputing dS,
    with the library's fixed scratch instead of a workspace (no device memory
    is allocated when dq, dk and dv are given)."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    for name, t, shp in (("q", q, (B, Hq, N, D)), ("k", k, (B, Hkv, N, D)),
                         ("v", v, (B, Hkv, N, D)), ("o", o, (B, Hq, N, D)),
                         ("dout", dout, (B, Hq, N, D))):
        _check(name, t, torch.bfloat16, shp)
    _check("lse", lse, torch.float32, (B, Hq, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check("dq", dq, torch.bfloat16, (B, Hq, N, D))
    _check("dk", dk, torch.bfloat16, (B, Hkv, N, D))
    _check("dv", dv, torch.bfloat16, (B, Hkv, N, D))
    rc = fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv,
                        N, D, causal, scale, _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd_noalloc")
    return dq, dk, dv


def forward_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool, scale: float, *,
                   out=None, lse=None, workspace=None):
    """O (bf16) and LSE (fp32) of a variable-length batch.

    q [Hq, total, D], k/v [Hkv, total, D] bf16 device tensors; cu_seqlens an
    int32 device tensor of B + 1 cumulative sequence starts.  Sequence b is
    rows cu_seqlens[b]:cu_seqlens[b+1] of every head.
    """
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be [H, total, D]")
    Hq, total, D = q.shape
    Hkv = k.shape[0]
    _check("q", q, torch.bfloat16, (Hq, total, D))
    _check("k", k, torch.bfloat16, (Hkv, total, D))
    _check("v", v, torch.bfloat16, (Hkv, total, D))
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must hold B + 1 >= 2 entries")
    B = cu_seqlens.numel() - 1
    _check("cu_seqlens", cu_seqlens, torch.int32, (B + 1,))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device)
    _check("out", out, torch.bfloat16, (Hq, total, D))
    _check("lse", lse, torch.float32, (Hq, total))
    if total == 0:
        return out, lse
    ws_bytes = fa_fwd_varlen_workspace_size(B, total)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       cu_seqlens.data_ptr(), B, Hq, Hkv, total, int(max_seqlen), D, causal,
                       scale, workspace.data_ptr(), workspace.numel(), _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_varlen")
    return out, lse


def forward_splitkv(q, k, v, causal: bool, scale: float, *, num_splits: int = 0, out=None,
                    lse=None, workspace=None):
    """Decode-shaped forward: q [B,Hq,Nq,D] over k/v [B,Hkv,Nk,D] (bf16 device
    tensors), keys split into num_splits ranges (0: automatic) and merged.
    Causal aligns the queries with the last Nq key positions."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check("q", q, torch.bfloat16, (B, Hq, Nq, D))
    _check("k", k, torch.bfloat16, (B, Hkv, Nk, D))
    _check("v", v, torch.bfloat16, (B, Hkv, Nk, D))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check("out", out, torch.bfloat16, (B, Hq, Nq, D))
    _check("lse", lse, torch.float32, (B, Hq, Nq))
    ws_bytes = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, Nq, Nk, D, causal, scale, num_splits, wptr, wn,
                        _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_splitkv")
    return out, lse


def backward_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen: int, causal: bool,
                    scale: float, *, deterministic: int = 0, workspace=None):
    """dQ, dK, dV (bf16) of forward_varlen; deterministic is 0 (atomic), 1
    (fixed order from stored dS blocks; every sequence at most max_seqlen
    long) or 2 (fixed order, recomputing dS)."""
    import torch
    Hq, total, D = q.shape
    Hkv = k.shape[0]
    for name, t, shp in (("q", q, (Hq, total, D)), ("k", k, (Hkv, total, D)),
                         ("v", v, (Hkv, total, D)), ("o", o, (Hq, total, D)),
                         ("dout", dout, (Hq, total, D))):
        _check(name, t, torch.bfloat16, shp)
    _check("lse", lse, torch.float32, (Hq, total))
    B = cu_seqlens.numel() - 1
    _check("cu_seqlens", cu_seqlens, torch.int32, (B + 1,))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if total == 0:
        return dq, dk, dv
    ws_bytes = fa_bwd_varlen_workspace_size(B, Hq, Hkv, total, max_seqlen, D, deterministic)
    if workspace is None:
        # A size of 0 marks an invalid argument: the call below then reports
        # which one (it checks the arguments before the workspace).
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    rc = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       cu_seqlens.data_ptr(), B, Hq, Hkv, total, int(max_seqlen), D, causal, scale,
                       workspace.data_ptr(), workspace.numel(), deterministic,
                       _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd_varlen")
    return dq, dk, dv


def forward_fp8(q, k, v, causal: bool, scale: float, signs=None, *, out=None, lse=None,
                workspace=None):
    """FP8 forward: O (bf16), LSE (fp32) for q [B,Hq,N,D], k/v [B,Hkv,N,D] bf16
    device tensors; signs an optional float32 device tensor of D values +-1
    (the Hadamard rotation's random signs)."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    _check("q", q, torch.bfloat16, (B, Hq, N, D))
    _check("k", k, torch.bfloat16, (B, Hkv, N, D))
    _check("v", v, torch.bfloat16, (B, Hkv, N, D))
    if signs is not None:
        _check("signs", signs, torch.float32, (D,))
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    ws_bytes = fa_fwd_fp8_workspace_size(B, Hq, Hkv, N, D)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    rc = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                    Hkv, N, D, causal, scale, signs.data_ptr() if signs is not None else None,
                    workspace.data_ptr(), workspace.numel(), _stream_handle(q.device))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_fp8")
    return out, lse
