"""Variable-length backward (packed sequences, device-side work lists) against
the fp64 oracle applied to each sequence on its own, in dQ modes 0 (atomic),
1 (fixed order from stored dS blocks) and 2 (fixed order, recomputing dS)."""
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


@pytest.mark.parametrize("mode", [0, 1, 2])
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


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_bwd_fixed_order_is_deterministic_and_equals_dense(D, mode):
    dev = require_gpu()
    B, H, N = 3, 4, 384
    say(f"varlen bwd mode {mode} vs dense mode {mode}, B{B} H{H} N{N} D{D} causal, x5 reruns")
    q, k, v, do = synth.generate(B, H, H, N, D, seed=4, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.forward(qd, kd, vd, True, scale)
    dense = fa.backward(qd, kd, vd, o, lse, dod, True, scale, deterministic=mode)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, D).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=dev)
    lse_p = lse.permute(1, 0, 2).reshape(H, B * N).contiguous()
    digests = set()
    for _ in range(5):
        got = fa.backward_varlen(pack(qd), pack(kd), pack(vd), pack(o), lse_p, pack(dod), cu, N,
                                 True, scale, deterministic=mode)
        h = hashlib.sha256()
        for t in got:
            h.update(t.cpu().view(torch.int16).numpy().tobytes())
        digests.add(h.hexdigest())
    torch.cuda.synchronize()
    assert len(digests) == 1
    for a, b in zip(dense, got):
        assert torch.equal(pack(a).cpu(), b.cpu())


@pytest.mark.parametrize("lens,max_seqlen", [([640, 17, 0, 300], 640), ([640, 17, 0, 300], 64)])
def test_varlen_bwd_stored_ds_region_bounds(lens, max_seqlen):
    # Mode 1 sizes each head's dS region from max_seqlen.  The call must stay
    # inside the workspace it asked for (a guard tail after the requested
    # bytes comes back unchanged), and dK, dV, which the fixed-order modes
    # form in the same main kernel in the same order, equal mode 2's bit for
    # bit.  With the true bound dQ matches the oracle; with a bound far below
    # the longest sequence (640 > 64) the region is too small and dQ is
    # unspecified.
    dev = require_gpu()
    Hq, Hkv, D = 4, 2, 128
    say(f"varlen bwd mode 1 region bounds lens={lens} max_seqlen={max_seqlen}")
    q, k, v, do, cu = synth.generate_varlen(lens, Hq, Hkv, D, seed=11, with_dout=True)
    qd, kd, vd, dod, cud = q.to(dev), k.to(dev), v.to(dev), do.to(dev), cu.to(dev)
    scale = 1.0 / math.sqrt(D)
    total = sum(lens)
    o, lse = fa.forward_varlen(qd, kd, vd, cud, max(lens), True, scale)
    ref = fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, max(lens), True, scale, deterministic=2)
    ws_bytes = fa.fa_bwd_varlen_workspace_size(len(lens), Hq, Hkv, total, max_seqlen, D, 1)
    assert ws_bytes > 0
    guard = 4096
    buf = torch.full((ws_bytes + guard,), 0x5A, dtype=torch.uint8, device=dev)
    dq, dk, dv = fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, max_seqlen, True, scale,
                                    deterministic=1, workspace=buf[:ws_bytes])
    torch.cuda.synchronize()
    assert bool((buf[ws_bytes:] == 0x5A).all()), "dS blocks written past the workspace"
    assert torch.equal(ref[1].cpu(), dk.cpu()) and torch.equal(ref[2].cpu(), dv.cpu())
    if max_seqlen < max(lens):
        return
    dq = dq.cpu()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(int(cu[b]), int(cu[b]) + n)
        rq, _, _ = oracle.attention_bwd(q[None, :, sl], k[None, :, sl], v[None, :, sl],
                                        do[None, :, sl], True, scale)
        check_grad(dq[None, :, sl], rq, f"seq {b} (len {n}) dQ")


def test_varlen_bwd_many_short_sequences_all_modes():
    # 3000 sequences (lengths 0..40, seeded): more than the 1024 threads of
    # the block-offset scan, so each of its threads sums a run of sequences,
    # and many zero-length ones.  Mode 1's dK, dV equal mode 2's bit for bit
    # (same main kernel), its dQ agrees with mode 2's up to the summation
    # order, and sampled sequences match the oracle in every mode.
    dev = require_gpu()
    g = torch.Generator().manual_seed(12)
    lens = torch.randint(0, 41, (3000,), generator=g).tolist()
    Hq, Hkv, D = 2, 1, 64
    say(f"varlen bwd {len(lens)} sequences of 0..40 tokens (total {sum(lens)}), modes 0, 1, 2")
    q, k, v, do, cu = synth.generate_varlen(lens, Hq, Hkv, D, seed=13, with_dout=True)
    qd, kd, vd, dod, cud = q.to(dev), k.to(dev), v.to(dev), do.to(dev), cu.to(dev)
    scale = 1.0 / math.sqrt(D)
    ms = max(lens)
    o, lse = fa.forward_varlen(qd, kd, vd, cud, ms, True, scale)
    res = {m: [t.cpu() for t in fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, ms, True, scale,
                                                    deterministic=m)] for m in (0, 1, 2)}
    torch.cuda.synchronize()
    assert torch.equal(res[1][1], res[2][1]) and torch.equal(res[1][2], res[2][2])
    d1, d2 = res[1][0].double(), res[2][0].double()
    assert ((d1 - d2).norm() / d2.norm()).item() < 5e-3
    pick = [b for b in torch.randperm(len(lens), generator=g).tolist() if lens[b] > 0][:12]
    for b in pick:
        n = lens[b]
        sl = slice(int(cu[b]), int(cu[b]) + n)
        rq, rk, rv = oracle.attention_bwd(q[None, :, sl], k[None, :, sl], v[None, :, sl],
                                          do[None, :, sl], True, scale)
        for m, (dq, dk, dv) in res.items():
            check_grad(dq[None, :, sl], rq, f"mode {m} seq {b} (len {n}) dQ")
            check_grad(dk[None, :, sl], rk, f"mode {m} seq {b} dK")
            check_grad(dv[None, :, sl], rv, f"mode {m} seq {b} dV")


def test_varlen_bwd_stored_ds_sequence_far_beyond_max_seqlen():
    # One 50000-token sequence with max_seqlen = 64 in mode 1: the dS region is
    # sized for 64-token sequences, and the sequence's block indices reach
    # past 2^32 bytes (ceil(50000/32)^2 blocks of 2 KiB).  Block offsets are
    # formed in 64 bits, so every block outside the region is neither written
    # nor read: the call completes, the guard tail after the workspace comes
    # back unchanged, and dK, dV (which do not use the stored blocks) equal
    # mode 2's.  dQ is unspecified here.
    dev = require_gpu()
    lens, Hq, Hkv, D = [50000], 1, 1, 64
    say(f"varlen bwd mode 1, one sequence of {lens[0]} tokens, max_seqlen 64")
    q, k, v, do, cu = synth.generate_varlen(lens, Hq, Hkv, D, seed=21, with_dout=True)
    qd, kd, vd, dod, cud = q.to(dev), k.to(dev), v.to(dev), do.to(dev), cu.to(dev)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward_varlen(qd, kd, vd, cud, lens[0], True, scale)
    ref = fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, lens[0], True, scale, deterministic=2)
    ws_bytes = fa.fa_bwd_varlen_workspace_size(1, Hq, Hkv, lens[0], 64, D, 1)
    assert ws_bytes > 0
    guard = 4096
    buf = torch.full((ws_bytes + guard,), 0x3C, dtype=torch.uint8, device=dev)
    dq, dk, dv = fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, 64, True, scale, deterministic=1,
                                    workspace=buf[:ws_bytes])
    torch.cuda.synchronize()
    assert bool((buf[ws_bytes:] == 0x3C).all()), "written past the workspace"
    assert torch.equal(ref[1].cpu(), dk.cpu()) and torch.equal(ref[2].cpu(), dv.cpu())
    assert bool(torch.isfinite(dq.float()).all())


@pytest.mark.parametrize("mode", [1, 2])
def test_varlen_bwd_workload_sampled(mode):
    # The benchmark's length mix (64 sequences, 65536 tokens, 16 heads, D=128,
    # causal) in the launch configuration the benchmark times: dQ rows (first,
    # middle, last of heads 0 and 15) of every sequence one by one, and the
    # full dQ, dK, dV of heads 0 and 15 for the shortest and the longest
    # sequence, against the oracle.
    dev = require_gpu()
    w = synth.VARLEN
    lens = synth.varlen_lengths(w["n_seqs"], w["total"], w["lo"], w["hi"])
    H, D = w["Hq"], w["D"]
    say(f"varlen bwd workload mode {mode}: {len(lens)} sequences, {sum(lens)} tokens, max {max(lens)}")
    q, k, v, do, cu = synth.generate_varlen(lens, H, H, D, seed=0, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod, cud = q.to(dev), k.to(dev), v.to(dev), do.to(dev), cu.to(dev)
    o, lse = fa.forward_varlen(qd, kd, vd, cud, max(lens), True, scale)
    dq, dk, dv = (t.cpu() for t in fa.backward_varlen(qd, kd, vd, o, lse, dod, cud, max(lens), True,
                                                      scale, deterministic=mode))
    torch.cuda.synchronize()
    got, ref = [], []
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        sl = slice(s0, s0 + n)
        rows = [(0, h, i) for h in (0, H - 1) for i in sorted({0, n // 2, n - 1})]
        ref.append(oracle.attention_bwd_dq_rows(q[None, :, sl], k[None, :, sl], v[None, :, sl],
                                                do[None, :, sl], True, scale, rows))
        got.append(torch.stack([dq[h, s0 + i] for (_, h, i) in rows]))
    check_grad(torch.cat(got), torch.cat(ref), f"sampled dQ rows of all {len(lens)} sequences")
    for b in (min(range(len(lens)), key=lambda i: lens[i]), max(range(len(lens)), key=lambda i: lens[i])):
        s0, n = int(cu[b]), lens[b]
        sl = slice(s0, s0 + n)
        for h in (0, H - 1):
            one = lambda t: t[None, h:h + 1, sl]
            rq, rk, rv = oracle.attention_bwd(one(q), one(k), one(v), one(do), True, scale)
            check_grad(one(dq), rq, f"seq {b} (len {n}) head {h} dQ")
            check_grad(one(dk), rk, f"seq {b} head {h} dK")
            check_grad(one(dv), rv, f"seq {b} head {h} dV")
