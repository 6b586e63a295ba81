"""Decode-shaped split-KV forward against the fp64 oracle.  With causal, query
i of Nq sees keys 0 .. Nk - Nq + i, so each query position is checked as a
non-causal one-query problem over that key prefix (the plain definition)."""
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_lse, check_o, require_gpu, say

pytestmark = pytest.mark.gpu


def reference(q, k, v, causal, scale):
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    if not causal:
        return oracle.attention_fwd(q, k, v, False, scale)
    os, ls = [], []
    for i in range(Nq):
        L = Nk - Nq + i + 1
        o, l = oracle.attention_fwd(q[:, :, i:i + 1].contiguous(), k[:, :, :L].contiguous(),
                                    v[:, :, :L].contiguous(), False, scale)
        os.append(o)
        ls.append(l)
    return torch.cat(os, dim=2), torch.cat(ls, dim=2)


def inputs(B, Hq, Hkv, Nq, Nk, D, seed):
    # Queries and keys from one draw of the dense generator (Nk rows), the
    # queries being the last Nq positions.
    q, k, v = synth.generate(B, Hq, Hkv, Nk, D, seed=seed)
    return q[:, :, Nk - Nq:].contiguous(), k, v


CASES = [
    (2, 32, 1, 1, 3000, 128, True, 0), (2, 32, 1, 1, 3000, 128, False, 7),
    (1, 16, 4, 5, 1000, 128, True, 0), (1, 16, 4, 5, 1000, 128, True, 1),
    (3, 8, 2, 3, 777, 64, True, 0), (1, 4, 4, 40, 40, 64, True, 0),
    (1, 8, 1, 2, 65, 128, True, 2), (1, 8, 8, 130, 300, 128, False, 0),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,causal,splits", CASES)
def test_splitkv_matches_oracle(B, Hq, Hkv, Nq, Nk, D, causal, splits):
    dev = require_gpu()
    auto = fa.fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, D)
    say(f"split-KV B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} D{D} causal={causal} "
        f"splits={splits or f'auto({auto})'}")
    q, k, v = inputs(B, Hq, Hkv, Nq, Nk, D, seed=Nk + Nq)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), causal, scale, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = reference(q, k, v, causal, scale)
    check_o(o.cpu(), ro, "O")
    check_lse(lse.cpu(), rl, "LSE")


def test_split_count_does_not_change_the_result_beyond_rounding():
    dev = require_gpu()
    B, Hq, Hkv, Nq, Nk, D = 1, 32, 1, 1, 8192, 128
    q, k, v = inputs(B, Hq, Hkv, Nq, Nk, D, seed=3)
    scale = 1.0 / math.sqrt(D)
    res = []
    for sp in (1, 2, 16, 128):
        o, lse = fa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), True, scale, num_splits=sp)
        res.append((o.cpu().double(), lse.cpu().double()))
    torch.cuda.synchronize()
    ro, rl = reference(q, k, v, True, scale)
    for o, l in res:
        check_o(o, ro, "O")
        check_lse(l, rl, "LSE")


def test_decode_workload_full():
    # The benchmark's decode workload, B16 Hq32 Hkv1 Nq1 Nk32768 D128 causal,
    # with the split count the library picks (as the benchmark runs it): every
    # output row against the oracle.
    dev = require_gpu()
    B, Hq, Hkv, Nq, Nk, D = 16, 32, 1, 1, 32768, 128
    splits = fa.fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, D)
    say(f"split-KV decode workload B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} D{D}, {splits} key ranges")
    g = torch.Generator().manual_seed(1)
    q = torch.randn((B, Hq, Nq, D), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Nk, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Nk, D), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), True, scale, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = reference(q, k, v, True, scale)
    check_o(o.cpu(), ro, "O")
    check_lse(lse.cpu(), rl, "LSE")
