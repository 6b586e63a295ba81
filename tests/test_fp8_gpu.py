"""FP8 forward against the quantization-aware oracle (oracle/fp8.py): the
oracle rotates and quantizes Q, K, V exactly as the method defines and
attends exactly on the dequantized values; what it does not model is the
kernel's rounding of P to e4m3.  That rounding changes each P by at most
2^-4 relative (half of e4m3's 2^-3 mantissa step; 256 P stays a normal e4m3
value down to P = 2^-14), so each output element moves by at most
2^-4 max_j |V_j| (the dequantized V): the per-element gate is
max abs <= 2^-4 max|V| + 1e-2.  Over a tensor: with independent rounding
errors e_j of RMS s, O_i = sum_j P_ij V_j / l_i moves by about
s sqrt(sum_j P_ij^2 V_j^2) / l_i, and for zero-mean V that is s |O_i|, so the
relative L2 error is about s, the RMS relative error of round-to-nearest with
3 mantissa bits (2^-3 / sqrt(12) times E[1/m] for m in [1, 2): about 2.6e-2).
The gate is the worst-case relative rounding 2^-4 = 6.25e-2.  LSE comes from
the fp32 P sums: <= 1e-3."""
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from oracle import fp8
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def check_fp8(o, lse, ro, rl, vmax, what):
    o = o.double()
    err = (o - ro).abs().max().item()
    rel = ((o - ro).norm() / ro.norm()).item()
    lerr = (lse.double() - rl).abs().max().item()
    say(f"  {what}: O max abs {err:.3e} (bound {2 ** -4 * vmax + 1e-2:.3e}), rel L2 {rel:.3e}, "
        f"LSE max abs {lerr:.3e}")
    assert err <= 2 ** -4 * vmax + 1e-2, what
    assert rel <= 2 ** -4, what
    assert lerr <= 1e-3, what


def run(q, k, v, causal, scale, signs):
    dev = require_gpu()
    o, lse = fa.forward_fp8(q.to(dev), k.to(dev), v.to(dev), causal, scale,
                            signs.to(dev) if signs is not None else None)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = [
    (1, 2, 2, 300, 128, True, True), (1, 2, 2, 300, 128, True, False),
    (2, 4, 1, 257, 128, False, True), (1, 2, 2, 640, 64, True, True),
    (1, 3, 3, 100, 64, False, False), (1, 2, 1, 1, 128, True, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,causal,rot", CASES)
def test_fp8_matches_quantized_oracle(B, Hq, Hkv, N, D, causal, rot):
    say(f"fp8 fwd B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal} rotation={rot}")
    q, k, v = synth.generate(B, Hq, Hkv, N, D, seed=N + D)
    signs = synth.hadamard_signs(D, seed=D) if rot else None
    scale = 1.0 / math.sqrt(D)
    o, lse = run(q, k, v, causal, scale, signs)
    ro, rl = fp8.attention_fwd_fp8(q, k, v, causal, scale, signs=signs)
    vmax = float(v.double().abs().max()) * 1.07   # dequantized V <= |V| (1 + 2^-4)
    check_fp8(o, lse, ro, rl, vmax, "vs quantized oracle")


def _outlier_inputs():
    # Q and K with three channels 30x larger than the rest: quantizing per
    # tile then wastes almost all of e4m3's range on them unless the rotation
    # spreads them over the head dimension first.
    B, H, N, D = 1, 2, 512, 128
    q, k, v = synth.generate(B, H, H, N, D, seed=21)
    q, k = q.float(), k.float()
    for c in (3, 40, 77):
        q[..., c] *= 30.0
        k[..., c] *= 30.0
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v, 1.0 / math.sqrt(D) / 10.0


def test_fp8_outlier_channels_match_rotated_oracle():
    # Element by element against the rotated, quantized oracle, on inputs
    # where the rotation matters: the unrotated oracle is more than twice the
    # relative-L2 gate away from the rotated one, so a kernel that skipped or
    # misplaced the rotation would fail the gate (its own P rounding moves it
    # by about 2.6e-2 at most).
    say("fp8 outlier channels B1 H2 N512 D128 causal, rotation on, vs rotated oracle")
    q, k, v, scale = _outlier_inputs()
    signs = synth.hadamard_signs(128, seed=5)
    ro, rl = fp8.attention_fwd_fp8(q, k, v, True, scale, signs=signs)
    uo, _ = fp8.attention_fwd_fp8(q, k, v, True, scale, signs=None)
    gap = ((uo - ro).norm() / ro.norm()).item()
    say(f"  rotated vs unrotated oracle: rel L2 {gap:.3e}")
    assert gap > 2 * 2 ** -4
    o, lse = run(q, k, v, True, scale, signs)
    vmax = float(v.double().abs().max()) * 1.07
    check_fp8(o, lse, ro, rl, vmax, "outliers vs rotated oracle")


def test_rotation_reduces_error_on_outlier_channels():
    # Q and K with a few channels 30x larger than the rest: quantizing per
    # tile then wastes almost all of e4m3's range on them.  The rotation
    # spreads them, so the FP8 result moves closer to exact attention.
    say("fp8 outliers: error vs exact attention with and without rotation")
    q, k, v, scale = _outlier_inputs()
    D = q.shape[-1]
    ro, _ = oracle.attention_fwd(q, k, v, True, scale)
    errs = {}
    for rot in (False, True):
        signs = synth.hadamard_signs(D, seed=5) if rot else None
        o, lse = run(q, k, v, True, scale, signs)
        errs[rot] = ((o.double() - ro).norm() / ro.norm()).item()
    say(f"  rel L2 vs exact: no rotation {errs[False]:.3e}, rotation {errs[True]:.3e}")
    assert errs[True] < errs[False]


def test_fp8_headline_shape_one_head():
    # B2 H16 N8192 D128 causal, the last (batch, head) checked in full against
    # the quantized oracle (quantization is per (batch, head) tile, so that
    # head's oracle needs only its own tensors).
    w = synth.WORKLOADS["causal_a"]
    say(f"fp8 fwd full size B{w.B} H{w.Hq} N{w.N} D{w.D} causal, head ({w.B - 1},{w.Hq - 1})")
    q, k, v = synth.generate_workload(w)
    signs = synth.hadamard_signs(w.D, seed=0)
    o, lse = run(q, k, v, True, w.scale, signs)
    b, h = w.B - 1, w.Hq - 1
    sl = lambda t: t[b:b + 1, h:h + 1].contiguous()
    ro, rl = fp8.attention_fwd_fp8(sl(q), sl(k), sl(v), True, w.scale, signs=signs)
    vmax = float(sl(v).double().abs().max()) * 1.07
    check_fp8(sl(o), sl(lse), ro, rl, vmax, "head vs quantized oracle")
