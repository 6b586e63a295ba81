"""Backward parity: dQ, dK, dV from the HIP kernels against the fp64 oracle, in
the three dQ modes (0 atomic, 1 fixed order from stored dS, 2 fixed order
recomputing dS); bitwise determinism across reruns for modes 1 and 2."""
import hashlib
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_grad, check_lse, check_o, check_o_rounding_bound, require_gpu, say

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, dout, causal, scale, deterministic, reps=1):
    dev = require_gpu()
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    o, lse = fa.forward(qd, kd, vd, causal, scale)
    outs = []
    for _ in range(reps):
        outs.append(fa.backward(qd, kd, vd, o, lse, dod, causal, scale, deterministic=deterministic))
    torch.cuda.synchronize()
    return [tuple(t.cpu() for t in r) for r in outs]


SMALL = [
    (1, 1, 1, 1, 64, True), (1, 1, 1, 1, 128, False), (1, 2, 2, 17, 64, True),
    (2, 2, 2, 100, 128, False), (1, 2, 2, 255, 128, True), (1, 2, 2, 257, 64, True),
    (1, 3, 3, 300, 128, True), (1, 4, 2, 200, 128, True), (1, 4, 1, 130, 64, False),
    (2, 2, 2, 513, 64, False), (1, 2, 2, 640, 128, True),
]


MODES = [0, 1, 2]


@pytest.mark.parametrize("deterministic", MODES)
@pytest.mark.parametrize("B,Hq,Hkv,N,D,causal", SMALL)
def test_small_shapes(B, Hq, Hkv, N, D, causal, deterministic):
    say(f"bwd small B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal} det={deterministic}")
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=N + D + 1, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    (dq, dk, dv), = run_bwd(q, k, v, do, causal, scale, deterministic)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, causal, scale)
    check_grad(dq, rq, "dQ")
    check_grad(dk, rk, "dK")
    check_grad(dv, rv, "dV")


def _digest(ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.int16).numpy().tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("mode", [1, 2])
def test_deterministic_small_repeat(mode):
    q, k, v, do = synth.generate(1, 4, 4, 1000, 128, seed=5, with_dout=True)
    say(f"bwd deterministic mode {mode} x10 B1 H4 N1000 D128 causal")
    runs = run_bwd(q, k, v, do, True, 1 / math.sqrt(128), mode, reps=10)
    digests = {_digest(r) for r in runs}
    assert len(digests) == 1


# Whole heads compared element by element at full size: the first and last
# (batch, head) and two between them.
FULL_HEADS = [(0, 0), (0, 7), (1, 3), (1, 15)]


@pytest.mark.parametrize("name", ["bwd_d128", "bwd_d64"])
def test_full_size_config(name):
    w = synth.WORKLOADS[name]
    say(f"bwd full-size {name}: B{w.B} H{w.Hq} N{w.N} D{w.D} causal")
    q, k, v, do = synth.generate_workload(w)
    runs = {}
    for det in MODES:
        reps = 10 if det else 1
        res = run_bwd(q, k, v, do, w.causal, w.scale, det, reps=reps)
        if det:
            digests = {_digest(r) for r in res}
            say(f"  mode {det}: {len(digests)} distinct result(s) over {reps} reruns")
            assert len(digests) == 1
        runs[det] = res[0]
    # Both fixed-order modes form dK and dV in the same main kernel, in the
    # same order: identical bits.
    assert torch.equal(runs[1][1], runs[2][1]) and torch.equal(runs[1][2], runs[2][2])
    for b, h in FULL_HEADS:
        sl = lambda t: t[b:b + 1, h:h + 1]
        rq, rk, rv = oracle.attention_bwd(sl(q), sl(k), sl(v), sl(do), w.causal, w.scale)
        for det, (dq, dk, dv) in runs.items():
            tag = ("atomic", "stored dS", "recompute")[det]
            check_grad(sl(dq), rq, f"{tag} head ({b},{h}) dQ")
            check_grad(sl(dk), rk, f"{tag} head ({b},{h}) dK")
            check_grad(sl(dv), rv, f"{tag} head ({b},{h}) dV")
    # Every other head: dQ on sampled rows (each row's dQ needs only that
    # row's problem) and the key sum of dK, which is zero for every head
    # (rows of dS sum to zero).
    g = torch.Generator().manual_seed(3)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.Hq)
            for i in (0, w.N - 1, int(torch.randint(w.N, (1,), generator=g)))]
    rq = oracle.attention_bwd_dq_rows(q, k, v, do, w.causal, w.scale, rows)
    for det, (dq, dk, dv) in runs.items():
        tag = ("atomic", "stored dS", "recompute")[det]
        got = torch.stack([dq[b, h, i] for (b, h, i) in rows])
        check_grad(got, rq, f"{tag} sampled dQ rows ({len(rows)} over all heads)")
        s = dk.double().sum(dim=2).abs().max().item()
        scale_ref = dk.double().abs().sum(dim=2).max().item()
        assert s <= 2e-2 * scale_ref, (tag, s, scale_ref)


@pytest.mark.parametrize("deterministic", MODES)
@pytest.mark.parametrize("D", [64, 128])
def test_padding_keys_with_very_negative_scores(D, deterministic):
    # Non-causal, N not a multiple of any tile: the padding key rows read as
    # zero give the score 0, far above every real score (about -150 +- 20
    # here, so every row's LSE is below -90), and an unmasked padding key would
    # get P = exp(> 88.7) = inf in fp32 and dQ = inf * 0.  K's noise is as large
    # as its offset so that dQ = scale * sum_j dS_ij K_j is not a cancellation
    # of bf16-rounded terms.
    say(f"bwd padding keys, scores near -150, N130 D{D} det={deterministic}")
    B, H, N = 1, 2, 130
    g = torch.Generator().manual_seed(11)
    scale = 1.0 / math.sqrt(D)
    k = (1.0 + torch.randn(B, H, N, D, generator=g)).to(torch.bfloat16)
    q = (-150.0 / (D * scale) + 0.1 * torch.randn(B, H, N, D, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, H, N, D, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, N, D, generator=g).to(torch.bfloat16)
    (dq, dk, dv), = run_bwd(q, k, v, do, False, scale, deterministic)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, False, scale)
    check_grad(dq, rq, "dQ")
    check_grad(dk, rk, "dK")
    check_grad(dv, rv, "dV")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 8, 1, 300), (2, 16, 2, 1000)])
def test_grouped_heads_split_across_workgroups(B, Hq, Hkv, N, mode, D):
    # Few K/V tiles per head group: the warp-specialized main kernel (both
    # fixed-order modes) cuts each group's query heads into
    # parts (fp32 partial dK, dV summed in part order by a second pass).
    # Parity with the oracle, and bitwise repeatable.
    say(f"bwd grouped heads split B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal mode {mode} x3")
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=N + Hq, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    runs = run_bwd(q, k, v, do, True, scale, mode, reps=3)
    assert len({_digest(r) for r in runs}) == 1
    dq, dk, dv = runs[0]
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, True, scale)
    check_grad(dq, rq, "dQ")
    check_grad(dk, rk, "dK")
    check_grad(dv, rv, "dV")


@pytest.mark.parametrize("deterministic", MODES)
@pytest.mark.parametrize("D,scale", [(64, 0.05), (64, 0.2), (128, 0.04), (128, 0.15)])
def test_scale_other_than_inverse_sqrt_d(D, scale, deterministic):
    # The softmax scale is the caller's, not 1/sqrt(D): forward O and LSE and
    # the gradients of each dQ mode against the oracle at scales from 0.4x to
    # 1.7x of it (grouped heads, so the head-split partial dK path is
    # included).  Sharper scales are checked by test_sharp_softmax_scale.
    say(f"scale {scale} D{D} det={deterministic}: fwd + bwd B1 Hq4 Hkv2 N300 causal")
    dev = require_gpu()
    B, Hq, Hkv, N = 1, 4, 2, 300
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=17 + D, with_dout=True)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.forward(qd, kd, vd, True, scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, True, scale, deterministic=deterministic)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, True, scale)
    check_o(o.cpu(), o_ref, "O")
    check_lse(lse.cpu(), lse_ref, "LSE")
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, True, scale)
    check_grad(dq.cpu(), rq, "dQ")
    check_grad(dk.cpu(), rk, "dK")
    check_grad(dv.cpu(), rv, "dV")


@pytest.mark.parametrize("deterministic", MODES)
@pytest.mark.parametrize("D,scale", [(64, 0.3), (128, 0.25)])
def test_sharp_softmax_scale(D, scale, deterministic):
    # 2.4x and 2.8x the configured 1/sqrt(D): nearly one-hot rows, where the
    # bf16 rounding of P alone can move O by more than 1e-2 (measured
    # 1.26e-2 at 0.3, D = 64).  O is held to the bound derived from the
    # kernel's roundings of P and O (check_o_rounding_bound); LSE and the
    # gradients keep their gates.
    say(f"sharp scale {scale} D{D} det={deterministic}: fwd + bwd B1 Hq4 Hkv2 N300 causal")
    dev = require_gpu()
    B, Hq, Hkv, N = 1, 4, 2, 300
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=17 + D, with_dout=True)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.forward(qd, kd, vd, True, scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, True, scale, deterministic=deterministic)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, True, scale)
    o_absv, _ = oracle.attention_fwd(q, k, v.abs(), True, scale)
    check_o_rounding_bound(o.cpu(), o_ref, o_absv, "O")
    check_lse(lse.cpu(), lse_ref, "LSE")
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, True, scale)
    check_grad(dq.cpu(), rq, "dQ")
    check_grad(dk.cpu(), rk, "dK")
    check_grad(dv.cpu(), rv, "dV")


def test_grouped_heads_headline_size():
    # The benchmark's grouped-head workload, B2 Hq16 Hkv2 N8192 D128 causal,
    # stored-dS mode: K/V head 1 of batch 1 (query heads 8..15) in full
    # against the oracle, and dQ rows of every query head sampled one by one.
    B, Hq, Hkv, N, D = 2, 16, 2, 8192, 128
    say(f"bwd grouped heads B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal, stored dS")
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=2, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    [(dq, dk, dv)] = run_bwd(q, k, v, do, True, scale, 1)
    G = Hq // Hkv
    rq, rk, rv = oracle.attention_bwd(q[1:2, G:], k[1:2, 1:], v[1:2, 1:], do[1:2, G:], True, scale)
    check_grad(dq[1:2, G:], rq, "dQ of query heads 8..15, batch 1")
    check_grad(dk[1:2, 1:], rk, "dK of K/V head 1, batch 1")
    check_grad(dv[1:2, 1:], rv, "dV of K/V head 1, batch 1")
    g = torch.Generator().manual_seed(5)
    rows = [(b, h, i) for b in range(B) for h in range(Hq)
            for i in (0, N - 1, int(torch.randint(N, (1,), generator=g)))]
    ref = oracle.attention_bwd_dq_rows(q, k, v, do, True, scale, rows)
    got = torch.stack([dq[b, h, i] for (b, h, i) in rows])
    check_grad(got, ref, f"sampled dQ rows ({len(rows)} over all heads)")
