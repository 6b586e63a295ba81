"""Variable-length backward (packed sequences, device-side work lists) against
the fp64 oracle applied to each sequence on its own, in dQ modes 0 (atomic)
and 2 (fixed order, recomputing dS)."""
import hashlib
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_grad, require_gpu, say

pytestmark = pytest.mark.gpu


def run(lens, Hq, Hkv, D, causal, mode, seed, reps=1):
    dev = require_gpu()
    q, k, v, do, cu = synth.generate_varlen(lens, Hq, Hkv, D, seed=seed, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod, cud = q.to(dev), k.to(dev), v.to(dev), do.to(dev), cu.to(dev)
    ms = max(lens + [1])
    o, lse = fa.forward_varlen(qd, kd, vd, cud, ms, causal, scale)
    outs = [tuple(t.cpu() for t in fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, ms, causal,
                                                      scale, deterministic=mode))
            for _ in range(reps)]
    torch.cuda.synchronize()
    return q, k, v, do, cu, scale, outs


CASES = [
    ([1], 1, 1, 64, True), ([0, 5, 0], 2, 1, 64, False), ([127, 128, 129], 2, 2, 128, True),
    ([300, 17, 1, 640, 0, 256], 4, 2, 128, True), ([300, 17, 1, 640, 0, 256], 4, 4, 64, False),
    ([1000, 33], 2, 1, 128, False), ([700, 5, 1100], 2, 2, 64, True),
]


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("lens,Hq,Hkv,D,causal", CASES)
def test_varlen_bwd_matches_per_sequence_oracle(lens, Hq, Hkv, D, causal, mode):
    say(f"varlen bwd lens={lens} Hq{Hq} Hkv{Hkv} D{D} causal={causal} mode={mode}")
    q, k, v, do, cu, scale, [(dq, dk, dv)] = run(lens, Hq, Hkv, D, causal, mode, seed=len(lens) + D)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(int(cu[b]), int(cu[b]) + n)
        rq, rk, rv = oracle.attention_bwd(q[None, :, sl], k[None, :, sl], v[None, :, sl],
                                          do[None, :, sl], causal, scale)
        check_grad(dq[None, :, sl], rq, f"seq {b} (len {n}) dQ")
        check_grad(dk[None, :, sl], rk, f"seq {b} dK")
        check_grad(dv[None, :, sl], rv, f"seq {b} dV")


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_bwd_fixed_order_is_deterministic_and_equals_dense(D):
    dev = require_gpu()
    B, H, N = 3, 4, 384
    say(f"varlen bwd mode 2 vs dense mode 2, B{B} H{H} N{N} D{D} causal, x5 reruns")
    q, k, v, do = synth.generate(B, H, H, N, D, seed=4, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.forward(qd, kd, vd, True, scale)
    dense = fa.backward(qd, kd, vd, o, lse, dod, True, scale, deterministic=2)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, D).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=dev)
    lse_p = lse.permute(1, 0, 2).reshape(H, B * N).contiguous()
    digests = set()
    for _ in range(5):
        got = fa.backward_varlen(pack(qd), pack(kd), pack(vd), pack(o), lse_p, pack(dod), cu, N,
                                 True, scale, deterministic=2)
        h = hashlib.sha256()
        for t in got:
            h.update(t.cpu().view(torch.int16).numpy().tobytes())
        digests.add(h.hexdigest())
    torch.cuda.synchronize()
    assert len(digests) == 1
    for a, b in zip(dense, got):
        assert torch.equal(pack(a).cpu(), b.cpu())
