"""Fit the cubic used for 2^f on [0, 1) by the FMA-only exp2.

The exponential is split as 2^x = 2^n * 2^f with n = floor(x) and f = x - n,
and 2^f is replaced by p(f) = 1 + c1 f + c2 f^2 + c3 f^3 (hotelren
FlashAttention-4 summary, section 3.2; danialwang explainer, 巧招一 formula).
The pages give no coefficients, so they are fitted here: a discrete minimax
(Chebyshev) fit of the relative error |p(f)/2^f - 1| on a dense grid, solved
as a linear program, with p(0) = 1 held exactly so that the row maximum maps
to exactly 1.  Run it to print the coefficients that ``common.hpp`` holds.
"""
import numpy as np
from scipy.optimize import linprog


def fit(points: int = 20001):
    f = np.linspace(0.0, 1.0, points)
    t = np.exp2(f)
    rows = np.stack([f, f ** 2, f ** 3], axis=1) / t[:, None]
    rhs = (t - 1.0) / t
    ones = np.ones((points, 1))
    a_ub = np.vstack([np.hstack([rows, -ones]), np.hstack([-rows, -ones])])
    b_ub = np.concatenate([rhs, -rhs])
    res = linprog([0, 0, 0, 1], A_ub=a_ub, b_ub=b_ub, bounds=[(None, None)] * 4, method="highs")
    c1, c2, c3, err = res.x
    return c1, c2, c3, err


if __name__ == "__main__":
    c1, c2, c3, err = fit()
    for name, c in (("c1", c1), ("c2", c2), ("c3", c3)):
        print(f"{name} = {float(np.float32(c)):.9g}f  // {c:.17g}")
    print(f"max relative error on the grid: {err:.3e}")
