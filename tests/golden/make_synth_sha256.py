"""Writes synth_sha256.json: SHA-256 digests of the seeded synthetic inputs.

The inputs of every workload come from ``synth`` (a fresh CPU torch.Generator
seeded 0, fp32 randn in the order Q, K, V, dO, each rounded to bf16).  These
digests pin that recipe: a change to the draw order, the seed, the rounding or
the variant-(b) offsets changes them.  This script calls only ``synth``.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import synth  # noqa: E402

NAMES = ("tiny", "causal_b", "bwd_d128")


def digests(name):
    w = synth.WORKLOADS[name]
    ts = synth.generate_workload(w)
    return dict(zip(("q", "k", "v", "dout"), (synth.sha256(t) for t in ts)))


if __name__ == "__main__":
    doc = {"about": __doc__, "workloads": {n: digests(n) for n in NAMES}}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_sha256.json")
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    print(out)
