"""fa_bwd_noalloc, the backward that allocates nothing (its scratch is a fixed
buffer inside the library), against fa_bwd in the same dQ mode (2: fixed
order, recomputing dS) through the C ABI, on consecutive calls whose second
input is smaller than the first.

With one query head per K/V head the two entry points run the same kernels on
the same data, so the results must be bitwise equal.  With grouped heads
fa_bwd may split a group's heads over several workgroups and sum their fp32
partial dK, dV afterwards, while fa_bwd_noalloc sums the group in one
workgroup: dq stays bitwise equal, dk and dv are held to the relative L2 gate
of the gradients against fa_bwd and against the fp64 oracle."""
import math

import pytest
import torch

import exact_attention_98_amd as fa
import oracle
import synth
from tests.gpu_util import check_grad, rel_l2, require_gpu, say, RL2_GRAD

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, N, D, causal, seed):
    dev = require_gpu()
    q, k, v, do = synth.generate(B, Hq, Hkv, N, D, seed=seed, with_dout=True)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward(qd, kd, vd, causal, scale)
    return (q, k, v, do), (qd, kd, vd, o, lse, dod), scale


def _noalloc(t, B, Hq, Hkv, N, D, causal, scale):
    qd, kd, vd, o, lse, dod = t
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rc = fa.fa_bwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), dod.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), B, Hq, Hkv, N, D, int(causal), scale,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return dq, dk, dv


def _reference(t, B, Hq, Hkv, N, D, causal, scale):
    qd, kd, vd, o, lse, dod = t
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D, 2)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=qd.device)
    rc = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   dod.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, D,
                   int(causal), scale, ws.data_ptr(), ws_bytes, 2,
                   torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    return dq, dk, dv


def _bitwise(a, b, what):
    same = torch.equal(a.view(torch.int16), b.view(torch.int16))
    say(f"  {what}: bitwise equal = {same}")
    assert same, f"{what} differs from fa_bwd"


# (first call, second call with a smaller input)
PAIRS = [
    # one query head per K/V head: the headline size, then a ragged small one
    ((2, 16, 16, 8192, 128, True), (1, 2, 2, 300, 64, True)),
    # ragged non-causal, then a smaller D = 128 problem
    ((1, 3, 3, 777, 64, False), (1, 1, 1, 130, 128, True)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_fa_bwd_bitwise(first, second):
    for i, shape in enumerate((first, second)):
        B, Hq, Hkv, N, D, causal = shape
        say(f"noalloc call {i + 1}: B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal}")
        _, t, scale = _inputs(B, Hq, Hkv, N, D, causal, seed=N + 7 * i)
        got = _noalloc(t, *shape, scale)
        ref = _reference(t, *shape, scale)
        for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
            _bitwise(g, r, name)


def test_noalloc_grouped_heads():
    # fa_bwd splits each group's 4 query heads over 2 or 4 workgroups here
    # (few key tiles); fa_bwd_noalloc keeps them in one.
    for i, shape in enumerate(((1, 8, 2, 600, 128, True), (1, 4, 2, 200, 64, False))):
        B, Hq, Hkv, N, D, causal = shape
        say(f"noalloc grouped call {i + 1}: B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal}")
        cpu, t, scale = _inputs(B, Hq, Hkv, N, D, causal, seed=3 + i)
        got = _noalloc(t, *shape, scale)
        ref = _reference(t, *shape, scale)
        _bitwise(got[0], ref[0], "dQ")
        for g, r, name in zip(got[1:], ref[1:], ("dK", "dV")):
            d = rel_l2(g.cpu(), r.cpu())
            say(f"  {name}: relL2 vs fa_bwd = {d:.3e}")
            assert d <= RL2_GRAD
        rq, rk, rv = oracle.attention_bwd(*cpu, causal, scale)
        check_grad(got[0].cpu(), rq, "dQ vs oracle")
        check_grad(got[1].cpu(), rk, "dK vs oracle")
        check_grad(got[2].cpu(), rv, "dV vs oracle")


def test_noalloc_too_large_launches_nothing():
    require_gpu()
    rows = fa.BWD_NOALLOC_SCRATCH_BYTES // 8 + 1
    # Argument checks fail before the scratch lookup or any launch.
    rc = fa.fa_bwd_noalloc(1 << 36, 2 << 36, 3 << 36, 4 << 36, 5 << 36, 6 << 36, 7 << 36, 8 << 36,
                           9 << 36, 1, 1, 1, rows, 64, 1, 0.125, None)
    assert rc == fa.FA_ERR_SCRATCH


def test_noalloc_inside_a_captured_graph():
    # The use the entry point exists for: captured into a HIP graph (where no
    # allocation may happen) and replayed.  The first call on the device, made
    # before capture, looks up the scratch address; each replay, with eager
    # work and a synchronization between replays, must equal the eager result
    # bit for bit (dQ mode 2 is deterministic).
    B, Hq, Hkv, N, D, causal = 1, 4, 2, 320, 128, True
    say(f"noalloc graph capture B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal={causal}")
    _, t, scale = _inputs(B, Hq, Hkv, N, D, causal, seed=11)
    eager = _noalloc(t, B, Hq, Hkv, N, D, causal, scale)
    qd, kd, vd, o, lse, dod = t
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rc = fa.fa_bwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), dod.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), B, Hq, Hkv, N, D, int(causal), scale,
                                   side.cuda_stream)
            assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (dq, dk, dv):
            x.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        for g, r, name in zip((dq, dk, dv), eager, ("dQ", "dK", "dV")):
            _bitwise(g, r, f"replay {rep + 1} {name}")
        # eager work between replays, on the same scratch
        _noalloc(t, B, Hq, Hkv, N, D, causal, scale)
