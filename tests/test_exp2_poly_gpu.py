"""The forward's FMA-only exp2, evaluated on the device by the same inline
function the forward kernel uses (fa_exp2_poly_eval), equals a host evaluation
bit for bit.  The host follows the same steps, each rounded once to float32
from its exact value: clamp at -127, n = floor(x), f = x - n, three fused
multiply-adds in Horner order with the float32 coefficients, n added into the
exponent field, 0 for x < -127."""
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact_attention_98_amd as fa
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "exact_attention_98_amd", "csrc", "common.hpp")


def coeffs():
    text = open(HEADER).read()
    return [np.float32(float(re.search(n + r"\s*=\s*([0-9.eE+-]+)f", text).group(1)))
            for n in ("kExp2C1", "kExp2C2", "kExp2C3")]


def f32(q: Fraction) -> np.float32:
    """q rounded to the nearest float32, ties to even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    scale = Fraction(2) ** (23 - e)
    m = round(a * scale)  # ties to even
    return np.float32(sign * float(Fraction(m) / scale))


def host_exp2_poly(x: np.float32, c1, c2, c3) -> np.float32:
    if x < np.float32(-127.0):
        return np.float32(0.0)
    xc = max(x, np.float32(-127.0))
    n = np.floor(xc)
    f = f32(Fraction(float(xc)) - Fraction(float(n)))
    F = Fraction(float(f))
    p = f32(Fraction(float(c3)) * F + Fraction(float(c2)))
    p = f32(F * Fraction(float(p)) + Fraction(float(c1)))
    p = f32(F * Fraction(float(p)) + 1)
    bits = np.array([p], dtype=np.float32).view(np.int32)[0] + (np.int32(int(n)) << np.int32(23))
    return np.array([bits], dtype=np.int32).view(np.float32)[0]


def test_device_exp2_poly_matches_host_bitwise():
    dev = require_gpu()
    c1, c2, c3 = coeffs()
    g = np.random.default_rng(0)
    xs = np.concatenate([
        g.uniform(-130.0, 9.0, 12000), g.uniform(-2.0, 2.0, 6000),
        np.arange(-127, 10, dtype=np.float64),                       # integers: f = 0
        np.arange(-127, 10, dtype=np.float64) - 2.0 ** -20,          # f just below 1
        [-127.5, -127.0, -126.999, -0.5, 0.0, 1e-8, -1e-8, 7.9999995, 8.0, 8.5],
    ]).astype(np.float32)
    xs = np.concatenate([xs, np.float32([-np.inf])])
    say(f"exp2 poly: {xs.size} inputs, device vs host bit for bit")
    x_d = torch.from_numpy(xs).to(dev)
    y_d = torch.empty_like(x_d)
    rc = fa.fa_exp2_poly_eval(x_d.data_ptr(), y_d.data_ptr(), xs.size,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    got = y_d.cpu().numpy().view(np.int32)
    want = np.array([host_exp2_poly(x, c1, c2, c3) for x in xs], dtype=np.float32).view(np.int32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    # and it is exp2 within the fit's bound over the normal range
    ok = (xs >= -126.0) & np.isfinite(xs)
    rel = np.abs(y_d.cpu().numpy()[ok].astype(np.float64) / np.exp2(xs[ok].astype(np.float64)) - 1.0)
    assert rel.max() < 1.2e-4
