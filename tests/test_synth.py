"""The seeded synthetic inputs are reproducible: their SHA-256 digests equal
the ones tests/golden/make_synth_sha256.py recorded (written by calling only
the input generator), and the tiny workload has the stated shape and type."""
import json
import os

import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "synth_sha256.json")


def test_input_digests_match_recorded():
    with open(GOLDEN) as f:
        rec = json.load(f)["workloads"]
    for name, want in rec.items():
        ts = synth.generate_workload(synth.WORKLOADS[name])
        got = dict(zip(("q", "k", "v", "dout"), (synth.sha256(t) for t in ts)))
        assert got == want, name


def test_tiny_workload_shape_and_type():
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.generate_workload(w)
    for t in (q, k, v):
        assert t.dtype == torch.bfloat16 and t.shape == (1, 1, 256, 64)
    # N(0,1) draws: sample mean and variance near 0 and 1
    x = torch.cat([q.flatten(), k.flatten(), v.flatten()]).double()
    assert abs(x.mean().item()) < 0.05 and abs(x.var().item() - 1.0) < 0.05
