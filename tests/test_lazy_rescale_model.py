"""The conditional rescale with one final correction is exact.

An fp64 model of the forward's tiled loop (64-key tiles; rows grouped 32 to a
wave; a wave rescales all its rows to their own new max when any row's max
grew by more than tau; P = exp2(s c - m_ref) against the possibly stale m_ref;
O / l and LSE = (m_ref + log2 l) ln 2 at the end) must equal the oracle for
tau = 0 (rescale every tile), tau = 8 (the method; hotelren summary, section
3.3; danialwang explainer, 巧招二) and tau = 1e9 (only the first tile sets
m_ref).  The model also reports how often the rescale is taken.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

LOG2E = 1.0 / math.log(2.0)


def tiled_model(q, k, v, causal, scale, tau, bn=64, rows_per_wave=32):
    """Returns O, LSE (fp64) and the fraction of (wave, tile) steps that rescaled."""
    qd, kd, vd = (t.double().numpy()[0, 0] for t in (q, k, v))
    N, D = qd.shape
    c = scale * LOG2E
    O = np.zeros((N, D))
    LSE = np.zeros(N)
    taken = total = 0
    for w0 in range(0, N, rows_per_wave):
        rows = np.arange(w0, min(N, w0 + rows_per_wave))
        m_ref = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), D))
        kend = min(N, rows[-1] + 1) if causal else N
        for k0 in range(0, kend, bn):
            keys = np.arange(k0, min(kend, k0 + bn))
            s = qd[rows] @ kd[keys].T
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m_ref, s.max(axis=1) * c)
            total += 1
            if np.any(m_new > m_ref + tau):
                taken += 1
                alpha = np.where(np.isneginf(m_new), 1.0, np.exp2(m_ref - m_new))
                acc *= alpha[:, None]
                l *= alpha
                m_ref = m_new
            msub = np.where(np.isneginf(m_ref), 0.0, m_ref)
            p = np.exp2(s * c - msub[:, None])
            if tau < 64:
                assert np.all(p <= 2.0 ** tau * (1 + 1e-12))
            l += p.sum(axis=1)
            acc += p @ vd[keys]
        O[rows] = acc / l[:, None]
        LSE[rows] = (m_ref + np.log2(l)) / LOG2E
    return torch.from_numpy(O), torch.from_numpy(LSE), taken / max(total, 1)


@pytest.mark.parametrize("variant", ["a", "b"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tau", [0.0, 8.0, 1e9])
def test_lazy_rescale_equals_definition(tau, causal, variant):
    q, k, v = synth.generate(1, 1, 1, 300, 32, seed=3, variant=variant)
    scale = 1.0 / math.sqrt(32)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, causal, scale)
    o, lse, _ = tiled_model(q, k, v, causal, scale, tau)
    assert torch.allclose(o, o_ref[0, 0], rtol=0, atol=1e-12)
    assert torch.allclose(lse, lse_ref[0, 0], rtol=0, atol=1e-10)


def test_trigger_rate_reported():
    # Variant (a): after the first tile the max rarely grows by 2^8, so few
    # steps rescale; variant (b)'s key-position offset keeps raising the max.
    rates = {}
    for variant in ("a", "b"):
        q, k, v = synth.generate(1, 1, 1, 2048, 64, seed=0, variant=variant)
        _, _, rate = tiled_model(q, k, v, True, 1 / 8, 8.0)
        _, _, rate0 = tiled_model(q, k, v, True, 1 / 8, 0.0)
        rates[variant] = (rate, rate0)
        print(f"variant {variant}: rescale taken on {rate:.1%} of steps with tau=8 "
              f"(every step that grows the max with tau=0: {rate0:.1%})")
    assert rates["a"][0] < rates["b"][0]
    assert rates["a"][0] < rates["a"][1]


@pytest.mark.parametrize("variant", ["a", "b"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_bench_rescale_count_matches_the_model(tau, causal, variant):
    # bench.py counts the rescales on the headline inputs with a vectorised
    # form of the same decision (fp32 scores, as the kernel forms them); on
    # small inputs it must agree with this fp64 model step for step.
    import bench
    N, D = 300, 32
    q, k, v = synth.generate(1, 2, 1, N, D, seed=5, variant=variant)
    scale = 1.0 / math.sqrt(D)
    taken, total = bench.rescale_counts(q, k, causal, scale, tau, heads_per_chunk=1)
    want_taken = want_total = 0
    for h in range(2):
        _, _, rate = tiled_model(q[:, h:h + 1], k, v, causal, scale, tau)
        steps = sum(len(range(0, min(N, min(N, w0 + 32)) if causal else N, 64))
                    for w0 in range(0, N, 32))
        want_total += steps
        want_taken += round(rate * steps)
    assert total == want_total
    assert taken == want_taken
