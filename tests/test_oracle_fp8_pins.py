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
