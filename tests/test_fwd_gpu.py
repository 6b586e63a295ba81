"""Forward parity: the HIP kernel (through the C ABI) against the fp64 oracle."""
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_lse, check_o, require_gpu, say

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, causal, scale, poly=None):
    dev = require_gpu()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.forward(qd, kd, vd, causal, scale, exp_poly_quarters=poly)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SMALL = [
    (1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True), (1, 2, 1, 17, 64, True),
    (2, 2, 2, 100, 128, False), (1, 4, 2, 255, 128, True), (1, 2, 2, 257, 64, True),
    (1, 3, 1, 300, 128, False), (2, 4, 4, 513, 64, True), (1, 2, 2, 1000, 128, True),
    (1, 8, 1, 384, 128, True), (1, 1, 1, 129, 64, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,causal", SMALL)
def test_small_shapes(B, Hq, Hkv, N, D, causal):
    say(f"fwd small B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal}")
    q, k, v = synth.generate(B, Hq, Hkv, N, D, seed=N + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    check_o(o, o_ref, "O")
    check_lse(lse, lse_ref, "LSE")


@pytest.mark.parametrize("poly", [0, 1, 2])
@pytest.mark.parametrize("D,causal", [(64, True), (128, False), (128, True)])
def test_exp2_polynomial_share(poly, D, causal):
    say(f"fwd poly share {poly}/4 D{D} causal={causal}")
    q, k, v = synth.generate(1, 2, 1, 333, D, seed=3)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_fwd(q, k, v, causal, scale, poly=poly)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    check_o(o, o_ref, f"O poly{poly}")
    check_lse(lse, lse_ref, f"LSE poly{poly}")


def test_tiny_config():
    w = synth.WORKLOADS["tiny"]
    say("fwd tiny B1 H1 N256 D64")
    q, k, v = synth.generate_workload(w)
    o, lse = run_fwd(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, w.causal, w.scale)
    check_o(o, o_ref, "tiny O")
    check_lse(lse, lse_ref, "tiny LSE")


def test_causal_row_zero_and_bitwise_repeat():
    require_gpu()
    q, k, v = synth.generate(1, 4, 2, 700, 128, seed=11)
    o1, l1 = run_fwd(q, k, v, True, 0.088)
    o2, l2 = run_fwd(q, k, v, True, 0.088)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # Row 0 under the causal mask attends only to key 0: O_0 = V_0 exactly.
    assert torch.equal(o1[:, :, 0], v.repeat_interleave(2, 1)[:, :, 0])


def _sample_rows(B, H, N, n_random, seed):
    g = torch.Generator().manual_seed(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 129, N - 65, N - 2, N - 1]
    rows = []
    for t, i in enumerate(fixed):
        rows.append((t % B, (7 * t) % H, i))
    for _ in range(n_random):
        rows.append((int(torch.randint(B, (1,), generator=g)), int(torch.randint(H, (1,), generator=g)),
                     int(torch.randint(N, (1,), generator=g))))
    return rows


def _check_rows(o, lse, q, k, v, w, rows, tag):
    o_ref, lse_ref = oracle.attention_fwd_rows(q, k, v, w.causal, w.scale, rows)
    got_o = torch.stack([o[b, h, i] for (b, h, i) in rows])
    got_l = torch.stack([lse[b, h, i] for (b, h, i) in rows])
    check_o(got_o, o_ref, f"{tag} sampled O ({len(rows)} rows)")
    check_lse(got_l, lse_ref, f"{tag} sampled LSE")


def _check_head(o, lse, q, k, v, w, b, h, tag):
    G = w.Hq // w.Hkv
    o_ref, lse_ref = oracle.attention_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                                          v[b:b + 1, h // G:h // G + 1], w.causal, w.scale)
    check_o(o[b:b + 1, h:h + 1], o_ref, f"{tag} head ({b},{h}) O")
    check_lse(lse[b:b + 1, h:h + 1], lse_ref, f"{tag} head ({b},{h}) LSE")


@pytest.mark.parametrize("name", ["noncausal", "causal_a", "causal_b", "mqa", "gqa"])
def test_full_size_config(name):
    w = synth.WORKLOADS[name]
    say(f"fwd full-size {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} N{w.N} D{w.D} causal={w.causal}")
    q, k, v = synth.generate_workload(w)
    o, lse = run_fwd(q, k, v, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rows = _sample_rows(w.B, w.Hq, w.N, 48, seed=1)
    _check_rows(o, lse, q, k, v, w, rows, name)
    # Whole heads: the last (batch, head) of every config (at N = 32768 that
    # is a grouped head of the multi-query / grouped-query problems), and the
    # first one as well up to N = 8192.
    _check_head(o, lse, q, k, v, w, w.B - 1, w.Hq - 1, name)
    if w.N <= 8192:
        _check_head(o, lse, q, k, v, w, 0, 0, name)
