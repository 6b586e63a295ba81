"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU), builds it,
and runs the pin suite against that build in a subprocess: the suite must
fail.  This is how the pins are shown to be sensitive to a dropped term, a
wrong sign or index, or a swapped operand anywhere in the oracle.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "score_scale_dropped": ("s[j] = scale * dot(qi, K + (long)j * D, D);",
                            "s[j] = dot(qi, K + (long)j * D, D);"),
    "causal_off_by_one": ("return (i + 1 < Nk) ? i + 1 : Nk;", "return (i < Nk) ? i : Nk;"),
    "lse_missing_max": ("Lh[i] = m + log(l);", "Lh[i] = log(l);"),
    "gqa_head_map": ("const int hk = hq / G;", "const int hk = hq % Hkv;"),
    "dsoftmax_sign": ("s[j] * (dp[j] - delta)", "s[j] * (dp[j] + delta)"),
    "dq_scale_dropped": ("dqi[d] += scale * ds * kj[d];", "dqi[d] += ds * kj[d];"),
    "dk_scale_dropped": ("dkj[d] += scale * ds * qi[d];", "dkj[d] += ds * qi[d];"),
    "dv_uses_ds": ("dvj[d] += p * doi[d];", "dvj[d] += ds * doi[d];"),
    "dp_wrong_operand": ("dp[j] = dot(doi, V + (long)j * D, D);", "dp[j] = dot(doi, K + (long)j * D, D);"),
    "bwd_causal_mask": ("if (causal && j > i) continue;", "if (causal && j >= i) continue;"),
    "bwd_delta_from_dp_only": ("delta += s[j] * dp[j];", "delta += dp[j];"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(mutated), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
