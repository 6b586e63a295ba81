"""fp64 CPU oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path and never calls it.

The arithmetic lives in ``oracle.c`` (plain definition of softmax attention
and its gradients, fp64); this module builds it with gcc and marshals bf16
tensors to it.  Which passages each formula follows is stated at the top of
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (portable x86-64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # A test that checks the pins catch planted mistakes points this at a
        # deliberately broken build of oracle.c.
        path = os.environ.get("ORACLE_LIB_OVERRIDE", _LIB)
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        ci = ctypes.c_int
        lib.oracle_fwd.argtypes = [u16p, u16p, u16p, f64p, f64p, ci, ci, ci, ci, ci, ci, ci,
                                   ctypes.c_double]
        lib.oracle_fwd.restype = ci
        lib.oracle_fwd_f64.argtypes = [f64p, f64p, f64p, f64p, f64p, ci, ci, ci, ci, ci, ci, ci,
                                       ctypes.c_double]
        lib.oracle_fwd_f64.restype = ci
        lib.oracle_bwd.argtypes = [u16p, u16p, u16p, u16p, f64p, f64p, f64p, ci, ci, ci, ci, ci,
                                   ci, ci, ctypes.c_double]
        lib.oracle_bwd.restype = ci
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        lib.oracle_set_num_threads.argtypes = [ci]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls (timing only)."""
    _load().oracle_set_num_threads(int(n))


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype != torch.bfloat16:
        raise TypeError("oracle inputs must be bfloat16 tensors")
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy()).view(np.uint16)


def _ptr(a: np.ndarray, ty):
    return a.ctypes.data_as(ctypes.POINTER(ty))


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected [B, H, N, D] tensors")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    return B, Hq, Hkv, Nq, Nk, D


def attention_fwd(q, k, v, causal: bool, scale: float):
    """O (fp64 [B,Hq,Nq,D]) and LSE (fp64 [B,Hq,Nq], natural log) from bf16 q, k, v."""
    B, Hq, Hkv, Nq, Nk, D = _dims(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must match k")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    o = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Nq), dtype=np.float64)
    rc = _load().oracle_fwd(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                            _ptr(vb, ctypes.c_uint16), _ptr(o, ctypes.c_double),
                            _ptr(lse, ctypes.c_double), B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                            float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed ({rc})")
    return torch.from_numpy(o), torch.from_numpy(lse)


def attention_fwd_f64(q, k, v, causal: bool, scale: float):
    """As attention_fwd, for fp64 inputs (any real values, e.g. dequantized
    ones): O [B,Hq,Nq,D] and LSE [B,Hq,Nq], fp64."""
    B, Hq, Hkv, Nq, Nk, D = _dims(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must match k")
    qa, ka, va = (np.ascontiguousarray(t.detach().cpu().double().numpy()) for t in (q, k, v))
    o = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Nq), dtype=np.float64)
    rc = _load().oracle_fwd_f64(_ptr(qa, ctypes.c_double), _ptr(ka, ctypes.c_double),
                                _ptr(va, ctypes.c_double), _ptr(o, ctypes.c_double),
                                _ptr(lse, ctypes.c_double), B, Hq, Hkv, Nq, Nk, D,
                                int(bool(causal)), float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd_f64 failed ({rc})")
    return torch.from_numpy(o), torch.from_numpy(lse)


def attention_bwd(q, k, v, dout, causal: bool, scale: float):
    """dQ, dK, dV (fp64) from bf16 q, k, v, dO; P is recomputed in fp64."""
    B, Hq, Hkv, Nq, Nk, D = _dims(q, k)
    if tuple(v.shape) != tuple(k.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("inconsistent shapes")
    qb, kb, vb, db = _bits(q), _bits(k), _bits(v), _bits(dout)
    dq = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, Nk, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, Nk, D), dtype=np.float64)
    rc = _load().oracle_bwd(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                            _ptr(vb, ctypes.c_uint16), _ptr(db, ctypes.c_uint16),
                            _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                            _ptr(dv, ctypes.c_double), B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                            float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed ({rc})")
    return torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv)


def attention_fwd_rows(q, k, v, causal: bool, scale: float, rows):
    """O and LSE of selected query rows only, each computed on its own.

    ``rows`` is an iterable of (b, hq, i).  Row i of a causal problem attends
    to keys 0..i, so it is evaluated as a one-row non-causal problem over that
    key prefix.  Cost is O(N*D) per row, which lets full-size problems be
    checked on sampled rows.
    """
    B, Hq, Hkv, Nq, Nk, D = _dims(q, k)
    G = Hq // Hkv
    outs, lses = [], []
    for (b, hq, i) in rows:
        nk = min(i + 1, Nk) if causal else Nk
        hk = hq // G
        qi = q[b:b + 1, hq:hq + 1, i:i + 1, :]
        kk = k[b:b + 1, hk:hk + 1, :nk, :]
        vv = v[b:b + 1, hk:hk + 1, :nk, :]
        o, lse = attention_fwd(qi, kk, vv, False, scale)
        outs.append(o[0, 0, 0])
        lses.append(lse[0, 0, 0])
    return torch.stack(outs), torch.stack(lses)


def attention_bwd_dq_rows(q, k, v, dout, causal: bool, scale: float, rows):
    """dQ of selected query rows only, each computed on its own.

    dQ_i = scale * sum_j dS_ij K_j with dS_ij = P_ij (dP_ij - Delta_i) and
    Delta_i = sum_j P_ij dP_ij uses row i's scores, dO_i and the keys it sees,
    nothing of the other rows.  So row i is evaluated as a one-row problem
    over its key prefix (causal) or all keys, by the full backward above; the
    dK and dV of that problem are discarded.  ``rows`` is an iterable of
    (b, hq, i); returns fp64 [len(rows), D].
    """
    B, Hq, Hkv, Nq, Nk, D = _dims(q, k)
    G = Hq // Hkv
    outs = []
    for (b, hq, i) in rows:
        nk = min(i + 1, Nk) if causal else Nk
        hk = hq // G
        dq, _, _ = attention_bwd(q[b:b + 1, hq:hq + 1, i:i + 1, :], k[b:b + 1, hk:hk + 1, :nk, :],
                                 v[b:b + 1, hk:hk + 1, :nk, :], dout[b:b + 1, hq:hq + 1, i:i + 1, :],
                                 False, scale)
        outs.append(dq[0, 0, 0])
    return torch.stack(outs)
