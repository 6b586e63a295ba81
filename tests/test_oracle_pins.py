"""Pins for the fp64 oracle, checked against things other than the oracle itself.

* brute force: an independent pure-Python evaluation of softmax attention;
* finite differences: the oracle's gradients against central differences of
  the brute-force forward (so the backward is pinned to the forward);
* a library routine: PyTorch CPU fp64 scaled_dot_product_attention + autograd;
* closed forms and invariants: V = 1 (rows of P sum to one), key shift,
  Q = 0 (mean / prefix mean of V), causal row 0, N = 1, sum_j dK_j = 0,
  grouped heads against their expansion, key permutation (non-causal);
* a hand-derived worked example stored under tests/golden/.
"""
import json
import math
import os
import random

import pytest
import torch

import oracle
import synth
from tests import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nested(t):
    return t.double().tolist()


def _bf16(*shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 1, 1, 5, 3), (2, 2, 1, 7, 4), (1, 4, 2, 16, 8),
                                          (1, 2, 2, 1, 2), (1, 3, 3, 11, 5)])
def test_forward_matches_bruteforce(B, Hq, Hkv, N, D, causal):
    q = _bf16(B, Hq, N, D, seed=1)
    k = _bf16(B, Hkv, N, D, seed=2)
    v = _bf16(B, Hkv, N, D, seed=3)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    ob, lb = bruteforce.forward(_nested(q), _nested(k), _nested(v), causal, scale)
    assert torch.allclose(o, torch.tensor(ob, dtype=torch.float64), rtol=0, atol=1e-12)
    assert torch.allclose(lse, torch.tensor(lb, dtype=torch.float64), rtol=0, atol=1e-12)


def test_forward_unequal_lengths_matches_bruteforce():
    q = _bf16(1, 2, 3, 4, seed=4)
    k = _bf16(1, 1, 9, 4, seed=5)
    v = _bf16(1, 1, 9, 4, seed=6)
    o, lse = oracle.attention_fwd(q, k, v, False, 0.7)
    ob, lb = bruteforce.forward(_nested(q), _nested(k), _nested(v), False, 0.7)
    assert torch.allclose(o, torch.tensor(ob, dtype=torch.float64), rtol=0, atol=1e-12)
    assert torch.allclose(lse, torch.tensor(lb, dtype=torch.float64), rtol=0, atol=1e-12)


# ------------------------------------------------------- finite differences
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 1, 1, 4, 3), (1, 2, 1, 5, 2), (2, 2, 2, 3, 4)])
def test_gradients_match_finite_differences(B, Hq, Hkv, N, D, causal):
    q = _bf16(B, Hq, N, D, seed=11)
    k = _bf16(B, Hkv, N, D, seed=12)
    v = _bf16(B, Hkv, N, D, seed=13)
    do = _bf16(B, Hq, N, D, seed=14)
    scale = 0.9
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    base = {"q": _nested(q), "k": _nested(k), "v": _nested(v)}
    dnest = _nested(do)
    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        t = base[name]
        for idx in [(b, hh, i, d) for b in range(len(t)) for hh in range(len(t[0]))
                    for i in range(len(t[0][0])) for d in range(len(t[0][0][0]))]:
            b, hh, i, d = idx
            x0 = t[b][hh][i][d]
            vals = []
            for s in (+1, -1):
                t[b][hh][i][d] = x0 + s * h
                vals.append(bruteforce.loss(base["q"], base["k"], base["v"], dnest, causal, scale))
            t[b][hh][i][d] = x0
            fd = (vals[0] - vals[1]) / (2 * h)
            an = float(grad[idx])
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


# ------------------------------------------------------------ library routine
def _sdpa_reference(q, k, v, do, causal, scale):
    G = q.shape[1] // k.shape[1]
    qd = q.double().requires_grad_(True)
    kd = k.double().requires_grad_(True)
    vd = v.double().requires_grad_(True)
    ke = kd.repeat_interleave(G, dim=1)
    ve = vd.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qd, ke, ve, is_causal=causal, scale=scale)
    o.backward(do.double())
    s = scale * (qd.detach() @ ke.detach().transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.detach(), lse, qd.grad, kd.grad, vd.grad


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 2, 2, 97, 64), (2, 4, 1, 64, 32), (1, 4, 2, 130, 128)])
def test_matches_torch_sdpa_fp64(B, Hq, Hkv, N, D, causal):
    q = _bf16(B, Hq, N, D, seed=21)
    k = _bf16(B, Hkv, N, D, seed=22)
    v = _bf16(B, Hkv, N, D, seed=23)
    do = _bf16(B, Hq, N, D, seed=24)
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = _sdpa_reference(q, k, v, do, causal, scale)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    for a, r in ((o, o_ref), (lse, lse_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        assert torch.allclose(a, r, rtol=1e-10, atol=1e-10)


# ------------------------------------------------------ closed forms/invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    # With V = 1 every output row is sum_j P_ij, which must be exactly 1.
    q = _bf16(1, 2, 40, 16, seed=31, scale=3.0)
    k = _bf16(1, 2, 40, 16, seed=32, scale=3.0)
    v = torch.ones(1, 2, 40, 16, dtype=torch.bfloat16)
    o, _ = oracle.attention_fwd(q, k, v, causal, 0.25)
    assert torch.allclose(o, torch.ones_like(o), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # K <- K + 1 u^T adds scale * q_i . u to every score of row i: O, dQ, dK, dV
    # are unchanged and LSE_i moves by scale * q_i . u.  u is a power of two so
    # the shifted bf16 keys stay exact.
    N, D = 24, 8
    q = _bf16(1, 1, N, D, seed=41)
    k = (torch.randint(-8, 8, (1, 1, N, D), generator=torch.Generator().manual_seed(42)) / 4.0)
    v = _bf16(1, 1, N, D, seed=43)
    do = _bf16(1, 1, N, D, seed=44)
    u = torch.zeros(D)
    u[1], u[5] = 2.0, -1.0
    k0 = k.to(torch.bfloat16)
    k1 = (k + u).to(torch.bfloat16)
    assert torch.equal(k1.double() - k0.double(), u.double().expand_as(k1))
    scale = 0.5
    o0, l0 = oracle.attention_fwd(q, k0, v, causal, scale)
    o1, l1 = oracle.attention_fwd(q, k1, v, causal, scale)
    shift = scale * (q.double() @ u.double())
    assert torch.allclose(o0, o1, rtol=0, atol=1e-12)
    assert torch.allclose(l1 - l0, shift, rtol=0, atol=1e-12)
    g0 = oracle.attention_bwd(q, k0, v, do, causal, scale)
    g1 = oracle.attention_bwd(q, k1, v, do, causal, scale)
    for a, b in zip(g0, g1):
        assert torch.allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_values(causal):
    N, D = 33, 8
    q = torch.zeros(1, 1, N, D, dtype=torch.bfloat16)
    k = _bf16(1, 1, N, D, seed=51)
    v = _bf16(1, 1, N, D, seed=52)
    o, lse = oracle.attention_fwd(q, k, v, causal, 0.3)
    vd = v.double()[0, 0]
    if causal:
        counts = torch.arange(1, N + 1, dtype=torch.float64)
        expect = vd.cumsum(0) / counts[:, None]
        expect_lse = torch.log(counts)
    else:
        expect = vd.mean(0, keepdim=True).expand(N, D)
        expect_lse = torch.full((N,), math.log(N), dtype=torch.float64)
    assert torch.allclose(o[0, 0], expect, rtol=0, atol=1e-12)
    assert torch.allclose(lse[0, 0], expect_lse, rtol=0, atol=1e-12)


def test_causal_row_zero_is_first_value():
    N, D = 20, 16
    q = _bf16(1, 3, N, D, seed=61)
    k = _bf16(1, 3, N, D, seed=62)
    v = _bf16(1, 3, N, D, seed=63)
    scale = 0.125
    o, lse = oracle.attention_fwd(q, k, v, True, scale)
    assert torch.equal(o[0, :, 0], v.double()[0, :, 0])
    expect = scale * (q.double()[0, :, 0] * k.double()[0, :, 0]).sum(-1)
    assert torch.allclose(lse[0, :, 0], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key(causal):
    q = _bf16(2, 2, 1, 8, seed=71)
    k = _bf16(2, 2, 1, 8, seed=72)
    v = _bf16(2, 2, 1, 8, seed=73)
    do = _bf16(2, 2, 1, 8, seed=74)
    o, _ = oracle.attention_fwd(q, k, v, causal, 0.5)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.5)
    assert torch.equal(o, v.double())
    assert torch.count_nonzero(dq) == 0 and torch.count_nonzero(dk) == 0
    assert torch.equal(dv, do.double())


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    q = _bf16(1, 2, 30, 8, seed=81, scale=2.0)
    k = _bf16(1, 2, 30, 8, seed=82, scale=2.0)
    v = _bf16(1, 2, 30, 8, seed=83)
    do = _bf16(1, 2, 30, 8, seed=84)
    _, dk, _ = oracle.attention_bwd(q, k, v, do, causal, 0.4)
    assert dk.abs().max() > 1e-3
    assert torch.allclose(dk.sum(dim=2), torch.zeros(1, 2, 8, dtype=torch.float64), rtol=0,
                          atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_expanded(causal):
    B, Hq, Hkv, N, D = 2, 6, 2, 19, 8
    q = _bf16(B, Hq, N, D, seed=91)
    k = _bf16(B, Hkv, N, D, seed=92)
    v = _bf16(B, Hkv, N, D, seed=93)
    do = _bf16(B, Hq, N, D, seed=94)
    G = Hq // Hkv
    ke, ve = k.repeat_interleave(G, 1), v.repeat_interleave(G, 1)
    o, lse = oracle.attention_fwd(q, k, v, causal, 0.35)
    oe, lsee = oracle.attention_fwd(q, ke, ve, causal, 0.35)
    assert torch.allclose(o, oe, rtol=0, atol=1e-13) and torch.allclose(lse, lsee, rtol=0, atol=1e-13)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.35)
    dqe, dke, dve = oracle.attention_bwd(q, ke, ve, do, causal, 0.35)
    assert torch.allclose(dq, dqe, rtol=0, atol=1e-12)
    assert torch.allclose(dk, dke.view(B, Hkv, G, N, D).sum(2), rtol=0, atol=1e-12)
    assert torch.allclose(dv, dve.view(B, Hkv, G, N, D).sum(2), rtol=0, atol=1e-12)


def test_noncausal_key_permutation():
    q = _bf16(1, 1, 12, 8, seed=101)
    k = _bf16(1, 1, 12, 8, seed=102)
    v = _bf16(1, 1, 12, 8, seed=103)
    perm = torch.tensor(random.Random(5).sample(range(12), 12))
    o, lse = oracle.attention_fwd(q, k, v, False, 0.3)
    op, lsep = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], False, 0.3)
    assert torch.allclose(o, op, rtol=0, atol=1e-13) and torch.allclose(lse, lsep, rtol=0, atol=1e-13)


def test_sampled_rows_equal_full():
    q, k, v = synth.generate(1, 4, 2, 50, 16, seed=7)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, 0.25)
        rows = [(0, 0, 0), (0, 3, 49), (0, 1, 17), (0, 2, 33)]
        orow, lrow = oracle.attention_fwd_rows(q, k, v, causal, 0.25, rows)
        for n, (b, h, i) in enumerate(rows):
            assert torch.allclose(orow[n], o[b, h, i], rtol=0, atol=1e-13)
            assert abs(float(lrow[n] - lse[b, h, i])) < 1e-13


def test_sampled_dq_rows_equal_full():
    # dQ of a row from the one-row problem equals that row of the full
    # backward (itself pinned to brute force, finite differences and SDPA).
    q, k, v, do = synth.generate(2, 4, 2, 50, 16, seed=8, with_dout=True)
    for causal in (False, True):
        dq, _, _ = oracle.attention_bwd(q, k, v, do, causal, 0.25)
        rows = [(0, 0, 0), (1, 3, 49), (0, 1, 17), (1, 2, 33), (0, 3, 1)]
        got = oracle.attention_bwd_dq_rows(q, k, v, do, causal, 0.25, rows)
        for n, (b, h, i) in enumerate(rows):
            assert torch.allclose(got[n], dq[b, h, i], rtol=0, atol=1e-13)


# --------------------------------------------------------------- worked example
def test_golden_two_by_two():
    with open(os.path.join(GOLDEN, "two_by_two.json")) as f:
        g = json.load(f)
    q = torch.tensor(g["q"], dtype=torch.bfloat16).view(1, 1, 2, 2)
    k = torch.tensor(g["k"], dtype=torch.bfloat16).view(1, 1, 2, 2)
    v = torch.tensor(g["v"], dtype=torch.bfloat16).view(1, 1, 2, 2)
    for mode in ("noncausal", "causal"):
        o, lse = oracle.attention_fwd(q, k, v, mode == "causal", g["scale"])
        exp = g[mode]
        assert torch.allclose(o[0, 0], torch.tensor(exp["o"], dtype=torch.float64), rtol=0, atol=1e-15)
        assert torch.allclose(lse[0, 0], torch.tensor(exp["lse"], dtype=torch.float64), rtol=0,
                              atol=1e-15)
        dq, dk, dv = oracle.attention_bwd(q, k, v, torch.tensor(g["dout"], dtype=torch.bfloat16)
                                          .view(1, 1, 2, 2), mode == "causal", g["scale"])
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.allclose(t[0, 0], torch.tensor(exp[name], dtype=torch.float64), rtol=0,
                                  atol=1e-15), (mode, name)
