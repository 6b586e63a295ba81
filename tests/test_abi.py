"""The C ABI: library loads, exports every declared entry point, and rejects bad
arguments before launching anything.  No GPU is used: every call here fails an
argument check, which runs before any HIP call."""
import ctypes
import os
import re

import pytest

import exact_attention_98_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.load()
    names = _declared()
    assert set(names) == set(fa.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_strerror():
    assert fa.fa_strerror(0) == "success"
    for code in range(-7, 0):
        assert fa.fa_strerror(code) != "unknown status"
    assert fa.fa_strerror(-99) == "unknown status"


# Fake, well-separated, 256-byte aligned device addresses: never dereferenced,
# because each call below fails a host-side check first.
Q, K, V, O, L, DO, DQ, DK, DV, WS = [(i + 1) << 36 for i in range(10)]


def fwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, Hq=2, Hkv=1, N=64, D=128, causal=1, scale=0.1,
             stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                     a["D"], a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID), (dict(lse=None), fa.FA_ERR_INVALID),
    (dict(B=0), fa.FA_ERR_INVALID), (dict(N=0), fa.FA_ERR_INVALID), (dict(N=-5), fa.FA_ERR_INVALID),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID), (dict(Hkv=0), fa.FA_ERR_INVALID),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED), (dict(D=256), fa.FA_ERR_UNSUPPORTED),
    (dict(D=0), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID), (dict(scale=float("inf")), fa.FA_ERR_INVALID),
    (dict(scale=-1.0), fa.FA_ERR_UNSUPPORTED),
    (dict(q=Q + 2), fa.FA_ERR_ALIGN), (dict(o=O + 8), fa.FA_ERR_ALIGN),
    (dict(o=Q), fa.FA_ERR_INVALID), (dict(lse=O + 64), fa.FA_ERR_INVALID),
    (dict(B=1 << 10, Hq=1 << 10, Hkv=1 << 10, N=1 << 10, D=128), fa.FA_ERR_TOO_LARGE),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_fwd_ex_rejects_bad_share():
    assert fa.fa_fwd_ex(Q, K, V, O, L, 1, 1, 1, 64, 64, 0, 0.125, 3, None) == fa.FA_ERR_INVALID
    assert fa.fa_fwd_ex(Q, K, V, O, L, 1, 1, 1, 64, 64, 0, 0.125, -1, None) == fa.FA_ERR_INVALID


def test_workspace_size():
    B, H, N, D = 2, 16, 8192, 128
    s0 = fa.fa_bwd_workspace_size(B, H, H, N, D, 0)
    s1 = fa.fa_bwd_workspace_size(B, H, H, N, D, 1)
    s2 = fa.fa_bwd_workspace_size(B, H, H, N, D, 2)
    rows = 2 * B * H * N * 4                              # Delta and LSE * log2(e)
    assert s0 >= B * H * N * D * 4 + rows                 # atomic mode: fp32 dQ accumulator
    assert s1 >= B * H * N * N * 2 + rows                 # stored dS: bf16 32x32 blocks, N^2 per head
    assert rows <= s2 < s0 < s1                           # recompute: row constants only
    assert s0 % 256 == 0 and s1 % 256 == 0 and s2 % 256 == 0
    assert fa.fa_bwd_workspace_size(0, H, H, N, D, 0) == 0
    assert fa.fa_bwd_workspace_size(B, H, H, N, 80, 0) == 0
    assert fa.fa_bwd_workspace_size(B, H, H, N, D, 3) == 0    # no such mode
    assert fa.fa_bwd_workspace_size(B, H, H, N, D, -1) == 0
    # Stored dS addresses one head's blocks with 32-bit offsets.
    assert fa.fa_bwd_workspace_size(1, 1, 1, 46336, 64, 1) > 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 46400, 64, 1) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 46400, 64, 2) > 0
    # The atomic mode's fp32 accumulator of one head within 32-bit signed offsets.
    assert fa.fa_bwd_workspace_size(1, 1, 1, (1 << 22) - 1, 128, 0) > 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 1 << 22, 128, 0) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 1 << 22, 128, 2) > 0


def bwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=1, Hq=2, Hkv=2, N=100,
             D=64, causal=1, scale=0.125, ws=WS, wsb=1 << 30, det=0, stream=None)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                     a["dv"], a["B"], a["Hq"], a["Hkv"], a["N"], a["D"], a["causal"], a["scale"],
                     a["ws"], a["wsb"], a["det"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), fa.FA_ERR_INVALID), (dict(dv=None), fa.FA_ERR_INVALID),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=1024), fa.FA_ERR_WORKSPACE),
    (dict(ws=WS + 16), fa.FA_ERR_ALIGN), (dict(dk=DK + 4), fa.FA_ERR_ALIGN),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED), (dict(Hq=4, Hkv=3), fa.FA_ERR_INVALID),
    (dict(dq=Q), fa.FA_ERR_INVALID), (dict(dk=DV), fa.FA_ERR_INVALID),
    (dict(ws=DQ), fa.FA_ERR_INVALID), (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(det=3), fa.FA_ERR_INVALID), (dict(det=-1), fa.FA_ERR_INVALID),
    (dict(N=46400, det=1), fa.FA_ERR_TOO_LARGE),
    # Atomic mode: one head's fp32 dQ accumulator rows (N D 4 bytes) must stay
    # within 32-bit signed offsets.
    (dict(Hq=1, Hkv=1, N=1 << 22, D=128, det=0), fa.FA_ERR_TOO_LARGE),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def bwd_noalloc(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=1, Hq=2, Hkv=2, N=100,
             D=64, causal=1, scale=0.125, stream=None)
    a.update(kw)
    return fa.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                             a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["N"], a["D"],
                             a["causal"], a["scale"], a["stream"])


# Largest problem the fixed scratch holds: Delta and LSE * log2(e), 4 bytes
# per row each, each region rounded up to 256 bytes.
_NOALLOC_ROWS = fa.BWD_NOALLOC_SCRATCH_BYTES // 8


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID), (dict(dv=None), fa.FA_ERR_INVALID),
    (dict(lse=None), fa.FA_ERR_INVALID), (dict(dk=DK + 4), fa.FA_ERR_ALIGN),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED), (dict(Hq=4, Hkv=3), fa.FA_ERR_INVALID),
    (dict(dq=Q), fa.FA_ERR_INVALID), (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(B=1, Hq=1, Hkv=1, N=_NOALLOC_ROWS + 1), fa.FA_ERR_SCRATCH),
    (dict(B=4, Hq=32, Hkv=8, N=32768 + 1), fa.FA_ERR_SCRATCH),
])
def test_bwd_noalloc_rejects(kw, code):
    # Every case fails a host-side check, before the scratch lookup (no GPU needed).
    assert bwd_noalloc(**kw) == code


def test_bwd_stages_reject():
    ws = 1 << 30
    assert fa.fa_bwd_preprocess(None, DO, L, 1, 2, 2, 64, 64, WS, ws, 0, None) == fa.FA_ERR_INVALID
    assert fa.fa_bwd_preprocess(O, DO, None, 1, 2, 2, 64, 64, WS, ws, 0, None) == fa.FA_ERR_INVALID
    assert fa.fa_bwd_preprocess(O, DO, L, 1, 2, 2, 64, 64, WS, 16, 0, None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_preprocess(O, DO + 8, L, 1, 2, 2, 64, 64, WS, ws, 0, None) == fa.FA_ERR_ALIGN
    assert fa.fa_bwd_preprocess(O, DO, WS, 1, 2, 2, 64, 64, WS, ws, 0, None) == fa.FA_ERR_INVALID
    assert fa.fa_bwd_main(Q, K, V, DO, DK, DV, 1, 2, 2, 64, 96, 1, 0.1, WS, ws, 0, None) == \
        fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_main(Q, K, V, DO, DK, DK, 1, 2, 2, 64, 64, 1, 0.1, WS, ws, 0, None) == \
        fa.FA_ERR_INVALID
    assert fa.fa_bwd_main(Q, K, V, DO, K, DV, 1, 2, 2, 64, 64, 1, 0.1, WS, ws, 0, None) == \
        fa.FA_ERR_INVALID
    assert fa.fa_bwd_dq(Q, K, V, DO, WS, 1, 2, 2, 64, 64, 1, 0.1, WS, ws, 0, None) == \
        fa.FA_ERR_INVALID
    assert fa.fa_bwd_dq(Q, K, V, DO, DQ + 2, 1, 2, 2, 64, 64, 1, 0.1, WS, ws, 1, None) == \
        fa.FA_ERR_ALIGN
    assert fa.fa_bwd_dq(Q, K, V, DO, Q, 1, 2, 2, 64, 64, 1, 0.1, WS, ws, 1, None) == \
        fa.FA_ERR_INVALID


def fwdv(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, cu=DQ, B=3, Hq=2, Hkv=1, total=500, max_seqlen=300, D=128,
             causal=1, scale=0.1, ws=WS, wsb=1 << 20, stream=None)
    a.update(kw)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["Hq"],
                            a["Hkv"], a["total"], a["max_seqlen"], a["D"], a["causal"], a["scale"],
                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID), (dict(cu=None), fa.FA_ERR_INVALID),
    (dict(ws=None), fa.FA_ERR_INVALID), (dict(B=0), fa.FA_ERR_INVALID),
    (dict(total=-1), fa.FA_ERR_INVALID), (dict(max_seqlen=0), fa.FA_ERR_INVALID),
    (dict(max_seqlen=1 << 30), fa.FA_ERR_INVALID), (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID), (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(cu=DQ + 2), fa.FA_ERR_ALIGN), (dict(ws=WS + 16), fa.FA_ERR_ALIGN),
    (dict(wsb=64), fa.FA_ERR_WORKSPACE), (dict(o=Q), fa.FA_ERR_INVALID),
    (dict(ws=L), fa.FA_ERR_INVALID), (dict(cu=O + 64), fa.FA_ERR_INVALID),
    (dict(Hq=1 << 10, Hkv=1 << 10, total=1 << 14), fa.FA_ERR_TOO_LARGE),
])
def test_fwd_varlen_rejects(kw, code):
    assert fwdv(**kw) == code


def test_fwd_varlen_empty_batch_is_a_no_op():
    # total = 0: every check passes and nothing is launched (fake pointers).
    assert fwdv(total=0, max_seqlen=1) == fa.FA_OK


def test_varlen_workspace_size():
    assert fa.fa_fwd_varlen_workspace_size(0, 10) == 0
    assert fa.fa_fwd_varlen_workspace_size(2, -1) == 0
    # One (sequence, 128-query tile) pair of int32 per possible item, plus a header.
    assert fa.fa_fwd_varlen_workspace_size(4, 1000) >= (1000 // 128 + 4) * 8
    assert fa.fa_varlen_max_seqlen() >= 1 << 19


def fwds(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=8, Hkv=1, Nq=1, Nk=1000, D=128, causal=1,
             scale=0.1, splits=4, ws=WS, wsb=1 << 24, stream=None)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["Nq"], a["Nk"], a["D"], a["causal"], a["scale"], a["splits"],
                             a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID), (dict(Nq=0), fa.FA_ERR_INVALID),
    (dict(Nk=0), fa.FA_ERR_INVALID), (dict(Nq=20, Nk=10), fa.FA_ERR_INVALID),
    (dict(splits=-1), fa.FA_ERR_INVALID), (dict(splits=17), fa.FA_ERR_INVALID),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED), (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID), (dict(k=K + 8), fa.FA_ERR_ALIGN),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=100), fa.FA_ERR_WORKSPACE),
    (dict(ws=WS + 64), fa.FA_ERR_ALIGN), (dict(o=K), fa.FA_ERR_INVALID),
    (dict(ws=O), fa.FA_ERR_INVALID),
    (dict(Hkv=1 << 8, Hq=1 << 8, Nk=1 << 17), fa.FA_ERR_TOO_LARGE),
    # Several key ranges: the fp32 partial rows of one K/V group (G Nq D 4
    # bytes) within 32-bit signed offsets.
    (dict(Hq=1024, Hkv=1, Nq=4096, Nk=8192), fa.FA_ERR_TOO_LARGE),
])
def test_fwd_splitkv_rejects(kw, code):
    assert fwds(**kw) == code


def test_splitkv_sizes():
    # Non-causal allows more queries than keys; one range needs no workspace.
    assert fa.fa_fwd_splitkv_workspace_size(1, 8, 1, 20, 10, 64, 1) == 0
    s = fa.fa_fwd_splitkv_num_splits(1, 32, 1, 1, 32768, 128)
    assert 1 <= s <= 32768 // 64
    rows = 1 * 32 * 1
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 1, 1, 32768, 128, 8) >= rows * 8 * (128 + 1) * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 1, 1, 32768, 128, 0) == \
        fa.fa_fwd_splitkv_workspace_size(1, 32, 1, 1, 32768, 128, s)
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 1, 1, 100, 128, 3) == 0   # ceil(100/64) = 2 ranges max
    assert fa.fa_fwd_splitkv_workspace_size(1, 1024, 1, 4095, 8192, 128, 4) > 0
    assert fa.fa_fwd_splitkv_workspace_size(1, 1024, 1, 4096, 8192, 128, 4) == 0
    assert fa.fa_fwd_splitkv_workspace_size(1, 1024, 1, 4096, 8192, 128, 1) == 0   # one range: none needed


def bwdv(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, cu=(11 << 36), B=3, Hq=2,
             Hkv=1, total=500, max_seqlen=300, D=128, causal=1, scale=0.1, ws=WS, wsb=1 << 24,
             det=2, stream=None)
    a.update(kw)
    return fa.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                            a["dv"], a["cu"], a["B"], a["Hq"], a["Hkv"], a["total"],
                            a["max_seqlen"], a["D"], a["causal"], a["scale"], a["ws"], a["wsb"],
                            a["det"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), fa.FA_ERR_INVALID), (dict(cu=None), fa.FA_ERR_INVALID),
    (dict(det=-1), fa.FA_ERR_INVALID), (dict(det=3), fa.FA_ERR_INVALID),
    (dict(det=1, total=1 << 22, max_seqlen=32768), fa.FA_ERR_TOO_LARGE),
    # Mode 0: one head's fp32 dQ accumulator, total * D * 4 bytes, must stay
    # below 2^31 (32-bit signed offsets).
    (dict(det=0, total=1 << 22, max_seqlen=32768), fa.FA_ERR_TOO_LARGE),
    (dict(B=0), fa.FA_ERR_INVALID), (dict(max_seqlen=1 << 30), fa.FA_ERR_INVALID),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED), (dict(dq=DQ + 4), fa.FA_ERR_ALIGN),
    (dict(wsb=64), fa.FA_ERR_WORKSPACE), (dict(dk=DQ), fa.FA_ERR_INVALID),
    (dict(dv=K), fa.FA_ERR_INVALID), (dict(ws=L), fa.FA_ERR_INVALID),
])
def test_bwd_varlen_rejects(kw, code):
    assert bwdv(**kw) == code


def test_bwd_varlen_sizes_and_empty_batch():
    assert bwdv(total=0, max_seqlen=1) == fa.FA_OK
    assert bwdv(total=0, max_seqlen=1, det=0) == fa.FA_OK
    assert bwdv(total=0, max_seqlen=1, det=1) == fa.FA_OK
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, 500, 300, 128, 3) == 0
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, 500, 0, 128, 2) == 0
    s0 = fa.fa_bwd_varlen_workspace_size(3, 2, 1, 500, 300, 128, 0)
    s1 = fa.fa_bwd_varlen_workspace_size(3, 2, 1, 500, 300, 128, 1)
    s2 = fa.fa_bwd_varlen_workspace_size(3, 2, 1, 500, 300, 128, 2)
    assert s0 >= 2 * 500 * 128 * 4 and s2 < s0
    # Mode 1 adds, per query head, (ceil(total/32) + B) * ceil(max_seqlen/32)
    # dS blocks of 32 x 32 bf16.
    assert s1 >= s2 + 2 * (16 + 3) * 10 * 2048
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, 1 << 22, 32768, 128, 1) == 0
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, 1 << 22, 32768, 128, 2) > 0
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, 1 << 22, 32768, 128, 0) == 0
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 1, (1 << 22) - 1, 32768, 128, 0) > 0


def test_exp2_poly_eval_argument_checks():
    # Rejected before any launch (no GPU needed); n = 0 launches nothing.
    assert fa.fa_exp2_poly_eval(None, None, -1, None) == fa.FA_ERR_INVALID
    assert fa.fa_exp2_poly_eval(None, None, 4, None) == fa.FA_ERR_INVALID
    assert fa.fa_exp2_poly_eval(None, None, 0, None) == fa.FA_OK
