"""Pins of the FP8 part of the oracle (oracle/fp8.py): e4m3 rounding against a
library conversion and hand-checked values, the rotation's orthogonality and
score invariance, and the quantizers' error bounds."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import fp8


def test_e4m3_rounding_matches_torch_conversion():
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(200000, generator=g, dtype=torch.float64) * s
                   for s in (1e-3, 1e-2, 0.1, 1.0, 10.0, 100.0)])
    x = x[x.abs() <= 448]
    ours = fp8.e4m3_round(x.numpy())
    lib = x.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, lib)


@pytest.mark.parametrize("x,want", [
    (448.0, 448.0), (460.0, 448.0), (1000.0, 448.0), (-2000.0, -448.0),
    (2.0 ** -9, 2.0 ** -9), (2.0 ** -10, 0.0), (3 * 2.0 ** -10, 2.0 ** -8),
    (1.0 + 1 / 16, 1.0), (1.0 + 3 / 16, 1.25), (2.0 ** -6, 2.0 ** -6),
    (15 * 2.0 ** -10, 2.0 ** -6), (-1.0625, -1.0), (0.0, 0.0), (256.0, 256.0), (272.0, 256.0),
    (288.0, 288.0),
])
def test_e4m3_hand_checked_values(x, want):
    assert fp8.e4m3_round(np.array([x]))[0] == want


def test_fwht_is_orthonormal_and_an_involution():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(7, 128, generator=g, dtype=torch.float64).numpy()
    y = fp8.fwht(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=0, atol=1e-12)
    assert np.allclose(fp8.fwht(y), x, rtol=0, atol=1e-12)
    # Against the Sylvester matrix built independently.
    H = np.array([[1.0]])
    while H.shape[0] < 8:
        H = np.block([[H, H], [H, -H]])
    z = np.random.default_rng(0).standard_normal((3, 8))
    assert np.allclose(fp8.fwht(z), z @ H.T / math.sqrt(8), rtol=0, atol=1e-13)


def test_rotation_leaves_scores_and_attention_unchanged():
    q, k, v = synth.generate(1, 2, 1, 40, 64, seed=2)
    signs = torch.where(torch.rand(64, generator=torch.Generator().manual_seed(3)) < 0.5, -1.0, 1.0)
    qr = fp8.rotate(q.double().numpy(), signs.numpy())
    kr = fp8.rotate(k.double().numpy(), signs.numpy())
    s0 = q.double().numpy() @ np.swapaxes(k.double().numpy(), -1, -2)
    s1 = qr @ np.swapaxes(kr, -1, -2)
    assert np.allclose(s0, s1, rtol=0, atol=1e-11)
    o0, l0 = oracle.attention_fwd(q, k, v, True, 0.125)
    o1, l1 = fp8.attention_fwd_fp8(q, k, v, True, 0.125, signs=signs, quantize=False)
    assert torch.allclose(o0, o1, rtol=0, atol=1e-12) and torch.allclose(l0, l1, rtol=0, atol=1e-12)


def test_quantizers_error_bounds_and_scales():
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(1, 2, 150, 64, generator=g, dtype=torch.float64) * 3).numpy()
    x[0, 0, 7, 5] = 40.0      # an outlier in the first tile of head 0
    deq, codes, f = fp8.quantize_scaled(x)
    # Each tile's largest element maps to +-448 exactly; every code is e4m3.
    assert np.all(np.abs(codes).max(axis=(3, 4)) == 448.0)
    assert np.array_equal(fp8.e4m3_round(codes), codes)
    # Relative error of a normal code at most 2^-4 (half of the 2^-3 mantissa step).
    big = np.abs(x) >= f.repeat(64, axis=2)[:, :, :150, None] * 2.0 ** -6
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-15
    dv, vcodes, e = fp8.quantize_pow2(x)
    amax = np.abs(fp8._tiles(x)[0]).max(axis=(3, 4))
    assert np.all(amax / 2.0 ** e <= 448.0) and np.all(amax / 2.0 ** (e - 1) > 448.0)
    assert np.array_equal(dv, (vcodes * 2.0 ** e[..., None, None]).reshape(1, 2, -1, 64)[:, :, :150])


def test_fp8_attention_close_to_exact_on_plain_inputs():
    # The quantization error itself is visible but bounded: on N(0,1) inputs
    # the FP8 result is within a few percent of exact attention.
    q, k, v = synth.generate(1, 2, 2, 200, 64, seed=5)
    o0, l0 = oracle.attention_fwd(q, k, v, True, 0.125)
    o1, l1 = fp8.attention_fwd_fp8(q, k, v, True, 0.125)
    rel = ((o1 - o0).norm() / o0.norm()).item()
    assert 1e-4 < rel < 5e-2


def _spike_rows(rng, n, positions, scale_rows=448.0):
    """Rows of 64 with two spikes: +-448 at one position and +-a at another,
    a in {40, 96, 160, 224}.  Every value is an e4m3 code and every row's
    largest magnitude is 448, so a tile of such rows quantizes exactly at
    factor 1."""
    y = np.zeros((n, 64))
    for i in range(n):
        p1, p2 = rng.choice(positions, size=2, replace=False)
        y[i, p1] = scale_rows * rng.choice([-1.0, 1.0])
        y[i, p2] = rng.choice([40.0, 96.0, 160.0, 224.0]) * rng.choice([-1.0, 1.0])
    return y


@pytest.mark.parametrize("causal", [False, True])
def test_rotation_applied_before_quantization(causal):
    # Q and K are built as the inverse rotation of rows whose rotated form is
    # exactly representable: rotate(Q) = Y with Y made of e4m3 codes at a tile
    # factor of 1 (Q = fwht(Y) * signs, since the orthonormal transform is its
    # own inverse, and (448 +- a) / 8 is exact in bf16).  V holds values whose
    # power-of-two quantization is exact too.  Rotating first and then
    # quantizing therefore loses nothing, and the FP8 oracle must equal exact
    # attention on the bf16 inputs.  Quantizing Q and K as given (before the
    # rotation, or with no rotation) rounds (448 +- a) / 8 at a tile factor of
    # 448 / 84 and moves the result; both mistakes are built here from the
    # oracle's own parts and must be told apart.
    rng = np.random.default_rng(7)
    D, N = 64, 64
    signs = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    positions = np.array([0, 5, 17, 40])
    yq = _spike_rows(rng, N, positions)
    yk = _spike_rows(rng, N, positions)
    qd = fp8.fwht(yq) * signs
    kd = fp8.fwht(yk) * signs
    q = torch.from_numpy(qd).reshape(1, 1, N, D).to(torch.bfloat16)
    k = torch.from_numpy(kd).reshape(1, 1, N, D).to(torch.bfloat16)
    assert torch.equal(q.double()[0, 0], torch.from_numpy(qd)), "Q must be exact in bf16"
    assert torch.equal(k.double()[0, 0], torch.from_numpy(kd)), "K must be exact in bf16"
    vvals = np.array([-1.5, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 1.5])
    v = torch.from_numpy(rng.choice(vvals, size=(1, 1, N, D))).to(torch.bfloat16)
    scale = 2e-5  # scores Y_q . Y_k of up to ~2.2e5 -> a few units

    exact_o, exact_l = oracle.attention_fwd(q, k, v, causal, scale)
    o, lse = fp8.attention_fwd_fp8(q, k, v, causal, scale, signs=torch.from_numpy(signs))
    assert torch.allclose(o, exact_o, rtol=0, atol=1e-9)
    assert torch.allclose(lse, exact_l, rtol=0, atol=1e-9)

    # The two plausible mistakes, from the same building blocks.
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    vq = fp8.quantize_pow2(vn)[0]
    assert np.array_equal(vq, vn)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    quant_then_rot = oracle.attention_fwd_f64(
        t(fp8.rotate(fp8.quantize_scaled(qn)[0], signs)),
        t(fp8.rotate(fp8.quantize_scaled(kn)[0], signs)), t(vq), causal, scale)[0]
    no_rotation = oracle.attention_fwd_f64(t(fp8.quantize_scaled(qn)[0]),
                                           t(fp8.quantize_scaled(kn)[0]), t(vq), causal, scale)[0]
    for wrong in (quant_then_rot, no_rotation):
        assert (wrong - exact_o).abs().max().item() > 1e-3
