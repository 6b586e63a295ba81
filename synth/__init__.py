"""Seeded synthetic inputs for attention, shared by the oracle checks and the HIP path.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic.  Each workload draws from a fresh CPU ``torch.Generator``
seeded with ``seed`` (default 0), fp32 ``randn`` in the order Q, K, V, then dO,
each rounded to bfloat16 (round to nearest even).  The same host tensors are
given to the oracle and, copied, to the device.

Workloads (the pages measure long-sequence bf16 attention with no printed
shapes, so these stand in for them):

* ``tiny``       B1 H1 N256 D64, non-causal
* ``noncausal``  B4 H16 N2048 D128, non-causal
* ``causal``     B2 H16 N8192 D128, causal, variant "a" (i.i.d. N(0,1)) or
                 variant "b" (Q, K scaled by 3 with a key-position offset on
                 channel 0, so the running row max keeps climbing)
* ``mqa``/``gqa`` B1 Hq32 Hkv{1,8} N32768 D128, causal
* ``bwd``        B2 H16 N8192 D128 causal, and B2 H16 N16384 D64 causal
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    causal: bool
    variant: str = "a"
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def flops_fwd(self) -> float:
        """4*B*Hq*N^2*D, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        """Backward counted as 2.5x the forward."""
        return 2.5 * self.flops_fwd()


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 64, False),
    "noncausal": Workload("noncausal", 4, 16, 16, 2048, 128, False),
    "causal_a": Workload("causal_a", 2, 16, 16, 8192, 128, True, "a"),
    "causal_b": Workload("causal_b", 2, 16, 16, 8192, 128, True, "b"),
    "mqa": Workload("mqa", 1, 32, 1, 32768, 128, True),
    "gqa": Workload("gqa", 1, 32, 8, 32768, 128, True),
    "bwd_d128": Workload("bwd_d128", 2, 16, 16, 8192, 128, True, backward=True),
    "bwd_d64": Workload("bwd_d64", 2, 16, 16, 16384, 64, True, backward=True),
}


def generate(B: int, Hq: int, Hkv: int, N: int, D: int, *, seed: int = 0, variant: str = "a",
             with_dout: bool = False):
    """Return bf16 CPU tensors (q, k, v[, dout]) of shapes [B,Hq,N,D], [B,Hkv,N,D]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, Hq, N, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32)
    dout = torch.randn((B, Hq, N, D), generator=g, dtype=torch.float32) if with_dout else None
    if variant == "b":
        # Q and K scaled by 3; channel 0 carries a per-row slope (0.5 .. 1.375,
        # cycling every 8 rows) times the key position, so the scaled score
        # grows along the key axis at a row-dependent rate.
        q = q * 3.0
        k = k * 3.0
        i = torch.arange(N, dtype=torch.float32)
        q[..., 0] = 0.5 + (i % 8) / 8.0
        k[..., 0] = i
    elif variant != "a":
        raise ValueError(f"unknown variant {variant!r}")
    out = [q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)]
    if with_dout:
        out.append(dout.to(torch.bfloat16))
    return tuple(out)


def generate_workload(w: Workload, seed: int = 0):
    return generate(w.B, w.Hq, w.Hkv, w.N, w.D, seed=seed, variant=w.variant, with_dout=w.backward)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.int16).numpy().tobytes()).hexdigest()


def varlen_lengths(n_seqs: int, total: int, lo: int, hi: int, *, seed: int = 0) -> list:
    """A seeded mix of sequence lengths: log-uniform in [lo, hi], rescaled so
    they sum to exactly `total` (each kept >= 1)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = torch.rand(n_seqs, generator=g, dtype=torch.float64)
    raw = torch.exp(torch.log(torch.tensor(float(lo))) +
                    u * (torch.log(torch.tensor(float(hi))) - torch.log(torch.tensor(float(lo)))))
    lens = [max(1, int(x)) for x in (raw * (total / raw.sum())).tolist()]
    lens[-1] += total - sum(lens)
    if lens[-1] < 1:
        raise ValueError("lengths do not fit the total")
    return lens


def generate_varlen(lens, Hq: int, Hkv: int, D: int, *, seed: int = 0, with_dout: bool = False):
    """Packed variable-length inputs: q [Hq,total,D], k/v [Hkv,total,D] (and
    dout [Hq,total,D]) bf16 CPU tensors plus cu_seqlens int32 [B+1].  Values:
    fp32 randn in the order Q, K, V, dO, rounded to bf16, as for the dense
    workloads."""
    total = int(sum(lens))
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((Hq, total, D), generator=g, dtype=torch.float32)
    k = torch.randn((Hkv, total, D), generator=g, dtype=torch.float32)
    v = torch.randn((Hkv, total, D), generator=g, dtype=torch.float32)
    out = [q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)]
    if with_dout:
        out.append(torch.randn((Hq, total, D), generator=g, dtype=torch.float32).to(torch.bfloat16))
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    return tuple(out) + (cu,)


# Variable-length forward workload: 64 sequences, 65536 tokens in total,
# lengths log-uniform in [128, 8192] (seed 0), 16 heads, D = 128, causal.
VARLEN = {"n_seqs": 64, "total": 65536, "lo": 128, "hi": 8192, "Hq": 16, "Hkv": 16, "D": 128,
          "causal": True}


def varlen_flops_fwd(lens, Hq: int, D: int, causal: bool) -> float:
    """4 Hq len^2 D per sequence, halved under the causal mask."""
    f = sum(4.0 * Hq * n * n * D for n in lens)
    return f / 2 if causal else f


def hadamard_signs(D: int, *, seed: int = 0) -> torch.Tensor:
    """Random +-1 signs of the FP8 path's Hadamard rotation (float32 [D])."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0).to(torch.float32)
