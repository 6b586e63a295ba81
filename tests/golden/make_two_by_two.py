"""Writes two_by_two.json: a 2-query, 2-key, D=2 attention problem solved by hand.

The expected values are closed forms derived on paper from the definition
O = softmax(scale * Q K^T) V (scale = 1) and its gradients; this script only
evaluates them with ``math``.  It calls neither the oracle nor the GPU path.

Q = [[1,0],[0,2]], K = I, V = [[1,2],[3,4]], dO = I.  Scores S = [[1,0],[0,2]].
Let a = sig(1), b = sig(-1) (row 0 weights), c = sig(-2), e = sig(2) (row 1).
Non-causal:  O0 = [1+2b, 2+2b], O1 = [1+2e, 2+2e], LSE = [ln(1+E), ln(1+E^2)],
  dP = [[1,3],[2,4]], Delta = [1+2b, 2+2e], dS = [[-2ab, 2ab], [-2ce, 2ce]],
  dQ = dS K = [[-2ab, 2ab], [-2ce, 2ce]], dK = dS^T Q = [[-2ab, -4ce], [2ab, 4ce]],
  dV = P^T dO = [[a, c], [b, e]].
Causal (key j visible to row i iff j <= i): row 0 sees key 0 only, so
  O0 = V0 = [1,2], LSE0 = 1, dS row 0 = 0; row 1 is unchanged.
  dQ = [[0,0], [-2ce, 2ce]], dK = [[0, -4ce], [0, 4ce]], dV = [[1, c], [0, e]].
"""
import json
import math
import os


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


a, b, c, e = sig(1.0), sig(-1.0), sig(-2.0), sig(2.0)
E = math.e
doc = {
    "about": __doc__,
    "q": [[1, 0], [0, 2]], "k": [[1, 0], [0, 1]], "v": [[1, 2], [3, 4]], "dout": [[1, 0], [0, 1]],
    "scale": 1.0,
    "noncausal": {
        "o": [[1 + 2 * b, 2 + 2 * b], [1 + 2 * e, 2 + 2 * e]],
        "lse": [math.log(1 + E), math.log(1 + E * E)],
        "dq": [[-2 * a * b, 2 * a * b], [-2 * c * e, 2 * c * e]],
        "dk": [[-2 * a * b, -4 * c * e], [2 * a * b, 4 * c * e]],
        "dv": [[a, c], [b, e]],
    },
    "causal": {
        "o": [[1.0, 2.0], [1 + 2 * e, 2 + 2 * e]],
        "lse": [1.0, math.log(1 + E * E)],
        "dq": [[0.0, 0.0], [-2 * c * e, 2 * c * e]],
        "dk": [[0.0, -4 * c * e], [0.0, 4 * c * e]],
        "dv": [[1.0, c], [0.0, e]],
    },
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "two_by_two.json"), "w") as f:
    json.dump(doc, f, indent=1)
