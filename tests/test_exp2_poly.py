"""The FMA-only exp2 used for part of the forward's exponentials.

2^x = 2^n * p(f), n = floor(x), f = x - n, p a cubic (hotelren summary,
section 3.2; danialwang explainer, 巧招一).  The pages print no coefficients
(parity unpinned for their values); what is checked is the property that
matters: the relative error stays below bf16's half spacing with margin,
p(0) = 1 exactly, and masked inputs give exactly 0.
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "exact_attention_98_amd", "csrc", "common.hpp")


def coeffs():
    text = open(HEADER).read()
    vals = {}
    for name in ("kExp2C1", "kExp2C2", "kExp2C3"):
        m = re.search(name + r"\s*=\s*([0-9.eE+-]+)f", text)
        vals[name] = np.float32(float(m.group(1)))
    return vals["kExp2C1"], vals["kExp2C2"], vals["kExp2C3"]


def exp2_poly_f32(x):
    """Step-by-step float32 evaluation of the kernel's exp2_poly."""
    c1, c2, c3 = coeffs()
    x = np.asarray(x, dtype=np.float32)
    xc = np.maximum(x, np.float32(-127.0))
    n = np.floor(xc).astype(np.float32)
    f = (xc - n).astype(np.float32)
    p = (f * c3 + c2).astype(np.float32)
    p = (f * p + c1).astype(np.float32)
    p = (f * p + np.float32(1.0)).astype(np.float32)
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    out = bits.view(np.float32)
    return np.where(x < -127.0, np.float32(0.0), out)


def test_fraction_polynomial_error_bound():
    c1, c2, c3 = coeffs()
    f = np.linspace(0.0, 1.0, 2_000_001, endpoint=False)
    p = 1.0 + f * (float(c1) + f * (float(c2) + f * float(c3)))
    rel = np.abs(p / np.exp2(f) - 1.0)
    assert rel.max() < 9e-5           # the fit's bound is 8.6e-5
    assert rel.max() < 2.0 ** -9 / 4  # well below bf16's half spacing
    assert 1.0 + 0.0 * float(c1) == 1.0  # p(0) = 1 exactly (no constant term to round)


def test_fit_script_reproduces_coefficients():
    pytest.importorskip("scipy")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fit_exp2_poly", os.path.join(ROOT, "exact_attention_98_amd", "csrc", "fit_exp2_poly.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    c1, c2, c3, err = mod.fit()
    for a, b in zip((c1, c2, c3), coeffs()):
        assert abs(a - float(b)) < 1e-6
    assert err < 9e-5


def test_full_exp2_in_float32():
    x = np.concatenate([np.linspace(-126.0, 8.0, 1_000_001, dtype=np.float32),
                        np.float32([0.0, 1.0, -1.0, 8.0, -0.5, 7.999999])])
    got = exp2_poly_f32(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(got / ref - 1.0)
    assert rel.max() < 1.2e-4
    assert exp2_poly_f32(np.float32([0.0]))[0] == 1.0
    for k in range(-20, 9):
        assert exp2_poly_f32(np.float32([k]))[0] == np.float32(2.0 ** k)


def test_masked_and_underflow_inputs_give_zero():
    x = np.float32([-np.inf, -1e30, -200.0, -127.5])
    assert np.all(exp2_poly_f32(x) == 0.0)
