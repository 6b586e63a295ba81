"""Pure-Python brute-force attention forward, for tiny inputs only.

Written independently of the oracle: nested loops over Python floats,
``math.exp``/``math.log`` and ``math.fsum``.  It takes fp64 nested lists (not
bf16), so it can also be evaluated at perturbed points for finite differences.
Layout q[b][h][i][d], k/v[b][hk][j][d]; query head h reads K/V head h // G.
"""
import math


def forward(q, k, v, causal, scale):
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    o, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            hk = h // G
            Q, K, V = q[b][h], k[b][hk], v[b][hk]
            oh, lh = [], []
            for i in range(len(Q)):
                scores = []
                for j in range(len(K)):
                    if causal and j > i:
                        continue
                    scores.append((j, scale * math.fsum(Q[i][d] * K[j][d] for d in range(len(Q[i])))))
                if not scores:
                    oh.append([0.0] * len(Q[i]))
                    lh.append(-math.inf)
                    continue
                m = max(s for _, s in scores)
                w = [(j, math.exp(s - m)) for j, s in scores]
                z = math.fsum(x for _, x in w)
                oh.append([math.fsum(x / z * V[j][d] for j, x in w) for d in range(len(Q[i]))])
                lh.append(m + math.log(z))
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse


def loss(q, k, v, dout, causal, scale):
    """L = sum over every element of O * dO."""
    o, _ = forward(q, k, v, causal, scale)
    terms = []
    for b in range(len(o)):
        for h in range(len(o[b])):
            for i in range(len(o[b][h])):
                for d in range(len(o[b][h][i])):
                    terms.append(o[b][h][i][d] * dout[b][h][i][d])
    return math.fsum(terms)
