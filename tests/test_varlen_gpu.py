"""Variable-length forward (packed sequences, device-side longest-first work
list) against the fp64 oracle applied to each sequence on its own."""
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_lse, check_o, require_gpu, say

pytestmark = pytest.mark.gpu


def run(lens, Hq, Hkv, D, causal, seed):
    dev = require_gpu()
    q, k, v, cu = synth.generate_varlen(lens, Hq, Hkv, D, seed=seed)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max(lens + [1]),
                               causal, scale)
    torch.cuda.synchronize()
    return q, k, v, cu, scale, o.cpu(), lse.cpu()


CASES = [
    ([1], 1, 1, 64, True), ([0, 5, 0], 2, 1, 64, False), ([127, 128, 129], 2, 2, 128, True),
    ([300, 17, 1, 640, 0, 256], 4, 2, 128, True), ([300, 17, 1, 640, 0, 256], 4, 4, 64, False),
    ([1000, 33], 2, 1, 128, False), ([2048, 5, 700], 2, 2, 64, True),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,causal", CASES)
def test_varlen_matches_per_sequence_oracle(lens, Hq, Hkv, D, causal):
    say(f"varlen fwd lens={lens} Hq{Hq} Hkv{Hkv} D{D} causal={causal}")
    q, k, v, cu, scale, o, lse = run(lens, Hq, Hkv, D, causal, seed=len(lens) + D)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        s0 = int(cu[b])
        sl = slice(s0, s0 + n)
        ro, rl = oracle.attention_fwd(q[None, :, sl], k[None, :, sl], v[None, :, sl], causal, scale)
        check_o(o[None, :, sl], ro, f"seq {b} (len {n}) O")
        check_lse(lse[None, :, sl], rl, f"seq {b} LSE")


def test_equal_lengths_match_dense_forward_bitwise():
    # The same kernel body runs both; only the addressing and the order of
    # the work differ, so equal-length batches must agree bit for bit.
    dev = require_gpu()
    B, H, N, D = 3, 4, 384, 128
    say(f"varlen vs dense, B{B} H{H} N{N} D{D} causal")
    q, k, v = synth.generate(B, H, H, N, D, seed=9)
    scale = 1.0 / math.sqrt(D)
    od, ld = fa.forward(q.to(dev), k.to(dev), v.to(dev), True, scale)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, D).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32)
    ov, lv = fa.forward_varlen(pack(q).to(dev), pack(k).to(dev), pack(v).to(dev), cu.to(dev), N,
                               True, scale)
    torch.cuda.synchronize()
    assert torch.equal(pack(od.cpu()), ov.cpu())
    assert torch.equal(ld.cpu().permute(1, 0, 2).reshape(H, B * N), lv.cpu())


def test_varlen_workload_sampled_rows():
    # The benchmark's length mix (64 sequences, 65536 tokens, 16 heads, D=128,
    # causal): every sequence's first, middle and last rows of head 0 and the
    # last head, checked one by one against the oracle.
    dev = require_gpu()
    w = synth.VARLEN
    lens = synth.varlen_lengths(w["n_seqs"], w["total"], w["lo"], w["hi"])
    say(f"varlen workload: {len(lens)} sequences, {sum(lens)} tokens, max {max(lens)}")
    q, k, v, cu = synth.generate_varlen(lens, w["Hq"], w["Hkv"], w["D"], seed=0)
    scale = 1.0 / math.sqrt(w["D"])
    o, lse = fa.forward_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max(lens), True, scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        sl = slice(s0, s0 + n)
        rows = [(0, h, i) for h in (0, w["Hq"] - 1) for i in sorted({0, n // 2, n - 1})]
        ro, rl = oracle.attention_fwd_rows(q[None, :, sl], k[None, :, sl], v[None, :, sl], True,
                                           scale, rows)
        ref_o.append(ro)
        ref_l.append(rl)
        got_o.append(torch.stack([o[h, s0 + i] for (_, h, i) in rows]))
        got_l.append(torch.stack([lse[h, s0 + i] for (_, h, i) in rows]))
    check_o(torch.cat(got_o), torch.cat(ref_o), f"sampled O ({sum(len(x) for x in got_o)} rows)")
    check_lse(torch.cat(got_l), torch.cat(ref_l), "sampled LSE")


@pytest.mark.parametrize("direction", ["fwd", "bwd0", "bwd1", "bwd2"])
def test_overlapping_sequences_stay_inside_the_workspace(direction):
    # cu_seqlens = [0, T, 0, T]: sequences 0 and 2 both cover rows 0..T-1
    # (clamping keeps each inside the tensors but not apart), which lists 20
    # (sequence, 128-row tile) items against room for T/128 + B = 13.  The
    # work list must stop at its capacity: the library gets exactly the
    # workspace it asks for, inside a larger buffer whose tail is a guard
    # pattern that must come back unchanged.  (Results for overlapping
    # sequences are unspecified -- items past the capacity are not run, so
    # some output rows are never written; the call must complete and stay in
    # bounds.)
    dev = require_gpu()
    T, Hq, Hkv, D = 1280, 2, 1, 128
    say(f"varlen overlapping cu_seqlens [0,T,0,T] T={T} {direction}")
    g = torch.Generator().manual_seed(4)
    mk = lambda h: torch.randn(h, T, D, generator=g).to(torch.bfloat16).to(dev)
    q, k, v = mk(Hq), mk(Hkv), mk(Hkv)
    cu = torch.tensor([0, T, 0, T], dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    guard = 4096
    if direction == "fwd":
        ws_bytes = fa.fa_fwd_varlen_workspace_size(3, T)
    else:
        ws_bytes = fa.fa_bwd_varlen_workspace_size(3, Hq, Hkv, T, T, D, int(direction[-1]))
    assert ws_bytes > 0
    buf = torch.full((ws_bytes + guard,), 0xA5, dtype=torch.uint8, device=dev)
    ws = buf[:ws_bytes]
    if direction == "fwd":
        fa.forward_varlen(q, k, v, cu, T, True, scale, workspace=ws)
    else:
        o, lse = fa.forward_varlen(q, k, v, cu, T, True, scale)
        fa.backward_varlen(q, k, v, o, lse, mk(Hq), cu, T, True, scale,
                           deterministic=int(direction[-1]), workspace=ws)
    torch.cuda.synchronize()
    assert bool((buf[ws_bytes:] == 0xA5).all()), "work list written past the workspace"
