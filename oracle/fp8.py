"""FP8 forward, as the method defines it -- test infrastructure only.

Written from the hotdry article (the FP8 / "incoherent processing" passage of
its memory-access section): before the Q K^T product, Q and K are rotated by a
fast Walsh-Hadamard transform with random signs, which spreads outlier
channels over the whole head dimension; the rotation is orthogonal, so
(Q R)(K R)^T = Q K^T and the scores are unchanged in exact arithmetic.  The
tensors are then quantized to FP8 (OCP e4m3) with one scale per tile of 64
rows of each (batch, head) -- for Q and K the scale maps the tile's largest
magnitude to 448, the largest e4m3 value; for V it is the power of two at or
above that ratio (so that it can be applied exactly inside the matrix
product).  Attention is then exact (the fp64 definition of oracle.c) on the
dequantized values.  Only the quantization of the inputs is modelled; the
kernel's own rounding of P to e4m3 is not (as the bf16 kernel's rounding of P
to bf16 is not), and the tests bound it separately.

Everything here is fp64 numpy/torch on the CPU.  The random signs are an input
(the caller draws them), so the same signs reach the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

from . import attention_fwd_f64

E4M3_MAX = 448.0           # 1.75 * 2^8: exponent field 15, mantissa 110 (111 is NaN)
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
TILE = 64                  # rows per quantization tile


def e4m3_round(x):
    """Nearest e4m3 value of each element (round half to even), saturating at
    +-448.  fp64 in, fp64 out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    out = np.zeros_like(a)
    normal = a >= E4M3_MIN_NORMAL
    # Normal binade [2^e, 2^(e+1)): 8 steps of 2^(e-3).
    e = np.floor(np.log2(np.where(normal, a, 1.0)))
    q = 2.0 ** (e - 3)
    out[normal] = (np.rint(a[normal] / q[normal]) * q[normal])
    # Subnormals: multiples of 2^-9 below 2^-6 (the rounding may land on 2^-6).
    sub = ~normal
    out[sub] = np.rint(a[sub] / E4M3_SUBNORMAL_STEP) * E4M3_SUBNORMAL_STEP
    out = np.minimum(out, E4M3_MAX)
    return np.copysign(out, x)


def fwht(x):
    """Orthonormal Walsh-Hadamard transform along the last axis (length a power
    of two): butterflies (a, b) -> (a + b, a - b) at distances 1, 2, 4, ...,
    then 1/sqrt(n)."""
    x = np.array(x, dtype=np.float64, copy=True)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < n:
        y = x.reshape(x.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(x.shape)
        h *= 2
    return x / np.sqrt(n)


def rotate(x, signs):
    """x R with R = diag(signs) H / sqrt(D): each row's elements times the
    random signs, then the orthonormal transform."""
    s = np.asarray(signs, dtype=np.float64)
    return fwht(np.asarray(x, dtype=np.float64) * s)


def _tiles(x):
    """View [B, H, N, D] as [B, H, ceil(N/64), 64, D] (zero-padded)."""
    B, H, N, D = x.shape
    nt = (N + TILE - 1) // TILE
    pad = np.zeros((B, H, nt * TILE, D))
    pad[:, :, :N] = x
    return pad.reshape(B, H, nt, TILE, D), N


def quantize_scaled(x):
    """Q / K: per tile, inv = 448 / amax, codes = e4m3(x inv), dequantization
    factor amax / 448.  Returns (dequantized values, codes, factors)."""
    t, N = _tiles(np.asarray(x, dtype=np.float64))
    amax = np.abs(t).max(axis=(3, 4), keepdims=True)
    amax = np.where(amax > 0, amax, E4M3_MAX)        # an all-zero tile: factor 1
    codes = e4m3_round(t * (E4M3_MAX / amax))
    deq = codes * (amax / E4M3_MAX)
    B, H = t.shape[:2]
    return (deq.reshape(B, H, -1, t.shape[-1])[:, :, :N], codes,
            (amax / E4M3_MAX)[..., 0, 0])


def quantize_pow2(x):
    """V: per tile, factor 2^e with e the smallest integer such that
    amax / 2^e <= 448; codes = e4m3(x / 2^e).  Returns (dequantized values,
    codes, exponents e)."""
    t, N = _tiles(np.asarray(x, dtype=np.float64))
    amax = np.abs(t).max(axis=(3, 4), keepdims=True)
    e = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX)), 0.0)
    codes = e4m3_round(t * 2.0 ** -e)
    deq = codes * 2.0 ** e
    B, H = t.shape[:2]
    return deq.reshape(B, H, -1, t.shape[-1])[:, :, :N], codes, e[..., 0, 0].astype(np.int64)


def attention_fwd_fp8(q, k, v, causal: bool, scale: float, signs=None, quantize: bool = True):
    """O, LSE (fp64) of the FP8 forward: rotate Q and K with the given signs (if
    any), quantize Q, K, V per 64-row tile, attention on the dequantized
    values.  quantize=False keeps only the rotation (then the result is plain
    attention)."""
    qf = q.double().numpy()
    kf = k.double().numpy()
    vf = v.double().numpy()
    if signs is not None:
        s = np.asarray(signs.double().numpy() if hasattr(signs, "numpy") else signs)
        qf = rotate(qf, s)
        kf = rotate(kf, s)
    if quantize:
        qf = quantize_scaled(qf)[0]
        kf = quantize_scaled(kf)[0]
        vf = quantize_pow2(vf)[0]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return attention_fwd_f64(t(qf), t(kf), t(vf), causal, scale)
