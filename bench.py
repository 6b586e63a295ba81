#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

One step = the whole path over one batch: the forward (fa_fwd: O and LSE)
followed by the backward's three stages (fa_bwd_preprocess, fa_bwd_main,
fa_bwd_dq: dK, dV, dQ), at B=2, H=16, N=8192, D=128, causal, bf16,
on seeded synthetic N(0,1) inputs already resident in device memory.

FLOPs per step follow the usual attention convention: forward 4*B*H*N^2*D,
halved for causal; backward 2.5x the forward.  Every launch is bracketed by
HIP events on the stream it runs on, so per-kernel averages are measured live.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
METRIC = "attention fwd/bwd TFLOPS + % bf16 MFMA peak, B2 H16 N8K D128 causal"
KERNEL_SOURCES = {
    "fwd_kernel": ["exact_attention_98_amd/csrc/fwd_kernel.hip",
                   "exact_attention_98_amd/csrc/common.hpp"],
    "bwd_ws_kernel": ["exact_attention_98_amd/csrc/bwd_kernels.hip",
                      "exact_attention_98_amd/csrc/common.hpp"],
    "bwd_atomic_kernel": ["exact_attention_98_amd/csrc/bwd_kernels.hip",
                          "exact_attention_98_amd/csrc/common.hpp"],
    "bwd_dq_kernel": ["exact_attention_98_amd/csrc/bwd_kernels.hip",
                      "exact_attention_98_amd/csrc/common.hpp"],
    "bwd_dq_ds_kernel": ["exact_attention_98_amd/csrc/bwd_kernels.hip",
                         "exact_attention_98_amd/csrc/common.hpp"],
}
# dQ modes of the backward (the deterministic argument of fa_bwd) and the
# kernel that finishes dQ in each.
DQ_MODES = {"stored": 1, "recompute": 2, "atomic": 0}
DQ_KERNEL = {0: "bwd_dq_convert_kernel", 1: "bwd_dq_ds_kernel", 2: "bwd_dq_kernel"}
DQ_LABEL = {0: "atomic", 1: "fixed order from stored dS (deterministic)",
            2: "fixed order, dS recomputed (deterministic)"}


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel: str, dq_mode: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (and, for the backward, in the same
    dQ mode); otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        rec = json.load(f)
    if kernel != "fwd_kernel" and rec.get("dq_mode") != dq_mode:
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, n_heads: int):
    """The fp64 oracle, as it stands, on the first n_heads (batch 0) of the workload."""
    import oracle
    import synth
    q, k, v, do = synth.generate(1, n_heads, n_heads, w.N, w.D, seed=0, with_dout=True)
    t0 = time.perf_counter()
    oracle.attention_fwd(q, k, v, w.causal, w.scale)
    oracle.attention_bwd(q, k, v, do, w.causal, w.scale)
    dt = time.perf_counter() - t0
    flops = (w.flops_fwd() + w.flops_bwd()) * n_heads / (w.B * w.Hq)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 forward+backward of {n_heads} of the {w.B * w.Hq} (batch, head) "
                      f"slices (N={w.N}, D={w.D}, causal), {dt:.1f} s wall",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "tiny_single_thread": tiny_single_thread(), "per_config": cpu_per_config()}


def cpu_per_config() -> dict:
    """The fp64 oracle on a bounded sample of every workload the parity tests
    cover (all host threads): whole (batch, head) slices of each workload's
    shape, drawn like it (seed 0), forward only except for the backward
    workloads.  One query head of the multi-query / grouped N=32768 forward is
    the same computation for Hkv = 1 and 8, so it is timed once for both."""
    import oracle
    import synth
    samples = [("tiny", 1), ("noncausal", 4), ("causal_a", 2), ("causal_b", 2), ("mqa", 1),
               ("bwd_d64", 1)]
    out = {}
    for name, heads in samples:
        w = synth.WORKLOADS[name]
        q, k, v, do = synth.generate(1, heads, heads, w.N, w.D, seed=0, variant=w.variant,
                                     with_dout=True)
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, w.causal, w.scale)
        if w.backward:
            oracle.attention_bwd(q, k, v, do, w.causal, w.scale)
        dt = time.perf_counter() - t0
        per_head = (w.flops_fwd() + (w.flops_bwd() if w.backward else 0.0)) / (w.B * w.Hq)
        key = "mqa_gqa" if name == "mqa" else name
        out[key] = {"workload": f"B{w.B} Hq{w.Hq} Hkv{w.Hkv} N{w.N} D{w.D} "
                                f"{'causal' if w.causal else 'non-causal'}"
                                f"{' variant ' + w.variant if name.startswith('causal') else ''}",
                    "pass": "forward+backward" if w.backward else "forward",
                    "sample_heads": heads, "seconds": round(dt, 3),
                    "tflops": round(per_head * heads / dt / 1e12, 4)}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def tiny_single_thread() -> dict:
    """The oracle's forward on the tiny workload (B1 H1 N256 D64, non-causal)
    on one OpenMP thread (set through the oracle library, then restored)."""
    import oracle
    import synth
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.generate_workload(w)
    before = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        oracle.attention_fwd(q, k, v, w.causal, w.scale)
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, w.causal, w.scale)
        sec = time.perf_counter() - t0
        threads = oracle.num_threads()
    finally:
        oracle.set_num_threads(before)
    return {"seconds": round(sec, 4), "threads": threads, "gflops": round(w.flops_fwd() / sec / 1e9, 2)}


def rescale_counts(q, k, causal: bool, scale: float, tau: float, bn: int = 64,
                   rows_per_wave: int = 32, heads_per_chunk: int = 4):
    """How often the forward's conditional rescale is taken on these inputs.

    Follows the kernel's decision: per wave of `rows_per_wave` query rows and
    per `bn`-key tile that the wave can see, the candidate max of each row is
    max(m_ref, c * tile max of its scores), c = scale * log2(e); the wave
    rescales (every row moves to its candidate) when any row's candidate
    exceeds its m_ref by more than tau (log2 units).  Scores are formed the way
    the kernel forms them (bf16 inputs, fp32 products and sums), on the device
    the tensors live on.  Returns (steps taken, wave-tile steps).
    q: [B, Hq, N, D], k: [B, Hkv, N, D] bf16."""
    import torch
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    c = scale / math.log(2.0)
    nt = (N + bn - 1) // bn
    nw = (N + rows_per_wave - 1) // rows_per_wave
    taken = total = 0
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    for i in range(0, len(heads), heads_per_chunk):
        chunk = heads[i:i + heads_per_chunk]
        qs = torch.stack([q[b, h] for b, h in chunk]).float()
        ks = torch.stack([k[b, h // G] for b, h in chunk]).float()
        s = torch.matmul(qs, ks.transpose(1, 2).contiguous())   # [h, N, N] fp32
        if causal:
            s.masked_fill_(torch.ones(N, N, dtype=torch.bool, device=s.device).triu_(1), -math.inf)
        pad = nt * bn - N
        if pad:
            s = torch.nn.functional.pad(s, (0, pad), value=-math.inf)
        tmax = s.view(len(chunk), N, nt, bn).amax(-1) * c        # [h, N, nt]
        del s
        rpad = nw * rows_per_wave - N
        if rpad:
            tmax = torch.nn.functional.pad(tmax, (0, 0, 0, rpad), value=-math.inf)
        tmax = tmax.reshape(len(chunk), nw, rows_per_wave, nt)
        m_ref = torch.full(tmax.shape[:3], -math.inf, device=tmax.device)
        last_row = torch.clamp(torch.arange(nw, device=tmax.device) * rows_per_wave
                               + rows_per_wave - 1, max=N - 1)
        for kt in range(nt):
            if causal:
                visible = kt * bn <= last_row
            else:
                visible = torch.ones_like(last_row, dtype=torch.bool)
            m_new = torch.maximum(m_ref, tmax[..., kt])
            trig = (m_new > m_ref + tau).any(-1) & visible[None, :]
            m_ref = torch.where(trig[..., None], m_new, m_ref)
            taken += int(trig.sum())
            total += int(visible.sum()) * len(chunk)
    return taken, total


def rescale_report(torch, dev) -> dict:
    """Rescale rate of the forward on the long causal inputs (variants a and b)
    with the kernel's tiles (32-row waves, 64-key tiles), at tau = 8 and at
    tau = 0 (a rescale whenever a row max grows).  The hotelren summary
    (section 3.3) reports about 85% fewer rescales with tau = 8."""
    import synth
    out = {}
    for var in ("a", "b"):
        w = synth.WORKLOADS[f"causal_{var}"]
        q, k, _ = (t.to(dev) for t in synth.generate_workload(w))
        t8, n = rescale_counts(q, k, True, w.scale, 8.0)
        t0, _ = rescale_counts(q, k, True, w.scale, 0.0)
        out[f"variant_{var}"] = {"wave_tile_steps": n, "rescaled_tau8": t8, "rescaled_tau0": t0,
                                 "rate_tau8": round(t8 / n, 4), "rate_tau0": round(t0 / n, 4),
                                 "fewer_rescales_than_tau0": round(1 - t8 / max(t0, 1), 4)}
        del q, k
    out["pages_fewer_rescales"] = 0.85
    out["what"] = ("forward conditional rescale on the B2 H16 N8192 D128 causal inputs: (wave, "
                   "64-key tile) steps that rescaled with tau = 8 (the method) and with tau = 0; "
                   "the first tile of each wave always rescales")
    return out


def bench_varlen(fa, torch, dev, stream, reps: int = 20) -> dict:
    """Variable-length forward on the packed workload of synth.VARLEN (the
    work-list kernel included in the timed call)."""
    import synth
    w = synth.VARLEN
    lens = synth.varlen_lengths(w["n_seqs"], w["total"], w["lo"], w["hi"])
    q, k, v, cu = (t.to(dev) for t in synth.generate_varlen(lens, w["Hq"], w["Hkv"], w["D"]))
    scale = 1.0 / math.sqrt(w["D"])
    o = torch.empty_like(q)
    lse = torch.empty((w["Hq"], w["total"]), dtype=torch.float32, device=dev)
    wsb = fa.fa_fwd_varlen_workspace_size(len(lens), w["total"])
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream

    def call():
        rc = fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), cu.data_ptr(), len(lens), w["Hq"], w["Hkv"],
                              w["total"], max(lens), w["D"], w["causal"], scale, ws.data_ptr(),
                              wsb, sh)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_varlen: {fa.fa_strerror(rc)}")

    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    flops = synth.varlen_flops_fwd(lens, w["Hq"], w["D"], w["causal"])
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": f"{len(lens)} causal sequences, {w['total']} tokens "
                        f"(lengths {min(lens)}..{max(lens)}, log-uniform mix), "
                        f"H{w['Hq']} D{w['D']}",
            "us": round(us, 1), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_varlen_bwd(fa, torch, dev, stream, det: int = 2, reps: int = 10) -> dict:
    """Variable-length backward (fa_bwd_varlen: preprocess, both work lists,
    dK/dV and dQ passes) on the packed workload of synth.VARLEN, dQ mode det
    (1: fixed order from stored dS blocks; 2: fixed order, recomputing dS)."""
    import synth
    w = synth.VARLEN
    lens = synth.varlen_lengths(w["n_seqs"], w["total"], w["lo"], w["hi"])
    q, k, v, cu = (t.to(dev) for t in synth.generate_varlen(lens, w["Hq"], w["Hkv"], w["D"]))
    g = torch.Generator(device="cpu")
    g.manual_seed(1)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(dev)
    scale = 1.0 / math.sqrt(w["D"])
    B, Hq, Hkv, total, D = len(lens), w["Hq"], w["Hkv"], w["total"], w["D"]
    o = torch.empty_like(q)
    lse = torch.empty((Hq, total), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fws = torch.empty(fa.fa_fwd_varlen_workspace_size(B, total), dtype=torch.uint8, device=dev)
    wsb = fa.fa_bwd_varlen_workspace_size(B, Hq, Hkv, total, max(lens), D, det)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream
    rc = fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          cu.data_ptr(), B, Hq, Hkv, total, max(lens), D, w["causal"], scale,
                          fws.data_ptr(), fws.numel(), sh)
    if rc != 0:
        raise RuntimeError(f"fa_fwd_varlen: {fa.fa_strerror(rc)}")

    def call():
        rc = fa.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), cu.data_ptr(), B, Hq, Hkv, total, max(lens), D,
                              w["causal"], scale, ws.data_ptr(), wsb, det, sh)
        if rc != 0:
            raise RuntimeError(f"fa_bwd_varlen: {fa.fa_strerror(rc)}")

    for _ in range(2):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    flops = 2.5 * synth.varlen_flops_fwd(lens, Hq, D, w["causal"])
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": f"{B} causal sequences, {total} tokens (lengths {min(lens)}..{max(lens)}), "
                        f"H{Hq} D{D}, dQ mode {det}",
            "us": round(us, 1), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_grouped(fa, torch, dev, stream, Hkv: int = 2, reps: int = 10, warmup: int = 3) -> dict:
    """Grouped heads (Hq 16 over Hkv K/V heads) at the headline size: forward
    plus backward (stored-dS dQ mode; dK and dV summed over each group inside
    the main kernel)."""
    B, Hq, N, D = 2, 16, 8192, 128
    g = torch.Generator(device="cpu")
    g.manual_seed(2)
    q = torch.randn((B, Hq, N, D), generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn((B, Hkv, N, D), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((B, Hkv, N, D), generator=g).to(torch.bfloat16).to(dev)
    do = torch.randn((B, Hq, N, D), generator=g).to(torch.bfloat16).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    det = 1
    wsb = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D, det)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    sh = stream.cuda_stream

    def call():
        rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, N, D, 1, scale, sh)
        if rc == 0:
            rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq,
                           Hkv, N, D, 1, scale, ws.data_ptr(), wsb, det, sh)
        if rc != 0:
            raise RuntimeError(f"grouped fwd+bwd: {fa.fa_strerror(rc)}")

    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    flops = 3.5 * 4.0 * B * Hq * N * N * D / 2   # forward 2 products + backward 5, causal
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": f"B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} causal, forward + backward (stored dS)",
            "us": round(us, 1), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_fp8(fa, torch, dev, stream, P, w, reps: int = 20) -> dict:
    """FP8 forward on the headline shape (same inputs as the bf16 step),
    rotation on; the timed call includes the quantize pass."""
    import synth
    B, Hq, Hkv, N, D = w.B, w.Hq, w.Hkv, w.N, w.D
    signs = synth.hadamard_signs(D).to(dev)
    wsb = fa.fa_fwd_fp8_workspace_size(B, Hq, Hkv, N, D)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    sh = stream.cuda_stream

    def call():
        rc = fa.fa_fwd_fp8(P["q"], P["k"], P["v"], o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, D,
                           1, w.scale, signs.data_ptr(), ws.data_ptr(), wsb, sh)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_fp8: {fa.fa_strerror(rc)}")

    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    tf = w.flops_fwd() / (us * 1e-6) / 1e12
    return {"workload": f"B{B} H{Hq} N{N} D{D} causal, e4m3, Hadamard rotation on "
                        "(quantize pass included)",
            "us": round(us, 1), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)}}


def bench_decode(fa, torch, dev, stream, reps: int = 50) -> dict:
    """Decode-shaped multi-query forward (split-KV + merge): one new query per
    sequence and head over a long K/V cache; bound by reading K and V."""
    import synth
    B, Hq, Hkv, Nq, Nk, D = 16, 32, 1, 1, 32768, 128
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    q = torch.randn((B, Hq, Nq, D), generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn((B, Hkv, Nk, D), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((B, Hkv, Nk, D), generator=g).to(torch.bfloat16).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    splits = fa.fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, D)
    wsb = fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, D, splits)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    sh = stream.cuda_stream

    def call():
        rc = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Nq, Nk, D, 1, scale, splits,
                               ws.data_ptr(), ws.numel(), sh)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_splitkv: {fa.fa_strerror(rc)}")

    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    # Algorithmic bytes: K and V once, Q and O once, LSE once.
    nbytes = 2 * B * Hkv * Nk * D * 2 + 2 * B * Hq * Nq * D * 2 + B * Hq * Nq * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} D{D} causal, {splits} key ranges",
            "us": round(us, 1), "tflops": round(4.0 * B * Hq * Nq * Nk * D / (us * 1e-6) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "bytes": nbytes}}


def bench_fwd_choices(fa, torch, dev, stream, P, w, reps: int = 20, rounds: int = 3) -> dict:
    """Forward design choices at the headline shape, each timed on the same
    stream in interleaved rounds (median of the per-round means):
    - the share of the exponentials computed by the FMA-only cubic instead of
      v_exp_f32 (fa_fwd_ex, 0, 1 or 2 quarters; 0 is what fa_fwd runs);
    - the conditional rescale under input variant (b), whose row maxima grow
      by more than tau on many tiles, against variant (a)."""
    import synth
    B, Hq, Hkv, N, D = w.B, w.Hq, w.Hkv, w.N, w.D
    sh = stream.cuda_stream
    o = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    wb = synth.WORKLOADS["causal_b"]
    qb, kb, vb = (t.to(dev) for t in synth.generate_workload(wb))

    def fwd(q, k, v, quarters):
        rc = fa.fa_fwd_ex(q, k, v, o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, D, 1, w.scale,
                          quarters, sh)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_ex: {fa.fa_strerror(rc)}")

    cases = {"poly_0": (P["q"], P["k"], P["v"], 0), "poly_1": (P["q"], P["k"], P["v"], 1),
             "poly_2": (P["q"], P["k"], P["v"], 2),
             "variant_b": (qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), 0)}
    times = {c: [] for c in cases}
    for _ in range(rounds):
        for c, args in cases.items():
            for _ in range(2):
                fwd(*args)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fwd(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            times[c].append(e0.elapsed_time(e1) / reps * 1e3)
    med = {c: sorted(t)[len(t) // 2] for c, t in times.items()}
    tf = lambda us: round(w.flops_fwd() / (us * 1e-6) / 1e12, 1)
    return {"workload": f"forward B{B} H{Hq} N{N} D{D} causal",
            "exp_poly_share": [{"quarters": qq, "us": round(med[f"poly_{qq}"], 1),
                                "tflops": tf(med[f"poly_{qq}"])} for qq in (0, 1, 2)],
            "lazy_rescale": {"variant_a_us": round(med["poly_0"], 1),
                             "variant_b_us": round(med["variant_b"], 1),
                             "variant_b_tflops": tf(med["variant_b"])}}


def bench_other_configs(fa, torch, dev, stream, reps: int = 5) -> dict:
    """Throughput at the other configurations the parity tests cover (inputs
    seeded N(0,1), drawn on the device): the non-causal forward B4 H16 N2048
    D128, the multi-query and grouped causal forwards B1 Hq32 Hkv1 / Hkv8
    N32768 D128, and the causal backward B2 H16 N16384 D64 in its three dQ
    modes (whole fa_bwd call)."""
    sh = stream.cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def timed(call):
        for _ in range(2):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    def line(name, us, flops):
        tf = flops / (us * 1e-6) / 1e12
        return {"workload": name, "us": round(us, 1), "tflops": round(tf, 1),
                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}

    out = {}
    for key, (B, Hq, Hkv, N, D, causal) in {
            "fwd_noncausal_B4H16N2048D128": (4, 16, 16, 2048, 128, False),
            "fwd_mqa_B1Hq32Hkv1N32768D128": (1, 32, 1, 32768, 128, True),
            "fwd_gqa_B1Hq32Hkv8N32768D128": (1, 32, 8, 32768, 128, True)}.items():
        q, k, v = rnd(B, Hq, N, D), rnd(B, Hkv, N, D), rnd(B, Hkv, N, D)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(D)

        def call():
            rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                           Hkv, N, D, int(causal), scale, sh)
            if rc != 0:
                raise RuntimeError(f"fa_fwd: {fa.fa_strerror(rc)}")

        flops = 4.0 * B * Hq * N * N * D / (2 if causal else 1)
        out[key] = line(f"forward B{B} Hq{Hq} Hkv{Hkv} N{N} D{D} {'causal' if causal else 'non-causal'}",
                        timed(call), flops)
        del q, k, v, o, lse
    B, H, N, D = 2, 16, 16384, 64
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    scale = 1.0 / math.sqrt(D)
    if fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N, D,
                 1, scale, sh) != 0:
        raise RuntimeError("fa_fwd failed")
    for det, tag in ((1, "stored"), (2, "recompute"), (0, "atomic")):
        wsb = fa.fa_bwd_workspace_size(B, H, H, N, D, det)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def call():
            rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H, N, D, 1,
                           scale, ws.data_ptr(), wsb, det, sh)
            if rc != 0:
                raise RuntimeError(f"fa_bwd: {fa.fa_strerror(rc)}")

        out[f"bwd_{tag}_B2H16N16384D64"] = line(
            f"backward B{B} H{H} N{N} D{D} causal, dQ mode {det} ({tag}), whole fa_bwd",
            timed(call), 2.5 * 4.0 * B * H * N * N * D / 2)
        del ws
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The first steps on a fresh process run slower (the first ten about 1.5x on average, while
    # the workspace is first touched and the clocks settle); 20 warm-up steps (about 45 ms) reach
    # the steady state that the timed steps then measure.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dq-mode", choices=list(DQ_MODES), default="stored",
                    help="backward dQ: fixed order from stored dS blocks (deterministic, "
                         "default), fixed order recomputing dS (deterministic, small "
                         "workspace), or atomic adds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the forward-choice, variable-length, grouped, decode, FP8 and "
                         "other-configuration measurements")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of MIB MiB (read MIB, write MIB) "
                         "so that memory-traffic counters can be scaled against known bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path runs on a single MI355X with no cross-GPU communication)",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import exact_attention_98_amd as fa
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    fa.load()
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["bwd_d128"]  # B2 H16 N8192 D128 causal, with dO
    B, Hq, Hkv, N, D = w.B, w.Hq, w.Hkv, w.N, w.D
    log(f"generating inputs B{B} H{Hq} N{N} D{D} causal (seed 0)")
    host = synth.generate_workload(w)
    input_sha = {n: synth.sha256(t) for n, t in zip(("q", "k", "v", "dout"), host)}
    q, k, v, do = (t.to(dev) for t in host)
    del host
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    det = DQ_MODES[args.dq_mode]
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D, det)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    P = dict(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=o.data_ptr(), lse=lse.data_ptr(),
             do=do.data_ptr(), dq=dq.data_ptr(), dk=dk.data_ptr(), dv=dv.data_ptr(),
             ws=ws.data_ptr())

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {fa.fa_strerror(rc)}")

    dq_name = DQ_KERNEL[det]
    # The fixed-order modes run the warp-specialized main kernel, the atomic mode its own.
    main_name = "bwd_atomic_kernel" if det == 0 else "bwd_ws_kernel"
    names = ["fwd_kernel", "bwd_pre_kernel", main_name, dq_name]

    def step(ev):
        ev[0].record(stream)
        check(fa.fa_fwd(P["q"], P["k"], P["v"], P["o"], P["lse"], B, Hq, Hkv, N, D, 1, w.scale, sh),
              "fa_fwd")
        ev[1].record(stream)
        check(fa.fa_bwd_preprocess(P["o"], P["do"], P["lse"], B, Hq, Hkv, N, D, P["ws"], ws_bytes,
                                   det, sh), "fa_bwd_preprocess")
        ev[2].record(stream)
        check(fa.fa_bwd_main(P["q"], P["k"], P["v"], P["do"], P["dk"], P["dv"], B, Hq, Hkv, N, D,
                             1, w.scale, P["ws"], ws_bytes, det, sh), "fa_bwd_main")
        ev[3].record(stream)
        check(fa.fa_bwd_dq(P["q"], P["k"], P["v"], P["do"], P["dq"], B, Hq, Hkv, N, D, 1, w.scale,
                           P["ws"], ws_bytes, det, sh), "fa_bwd_dq")
        ev[4].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {args.copy_calibration} MiB read + written")

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    evs = [events() for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per_kernel = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
                  for j, n in enumerate(names)}
    for n, t in per_kernel.items():
        log(f"  {n}: {t * 1e3:.1f} us/launch")

    def spread(us):
        """Median, min and max over the timed steps (microseconds)."""
        us = sorted(us)
        mid = len(us) // 2
        med = us[mid] if len(us) % 2 else 0.5 * (us[mid - 1] + us[mid])
        return {"median": round(med, 1), "min": round(us[0], 1), "max": round(us[-1], 1)}

    fwd_steps = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    bwd_steps = [e[1].elapsed_time(e[4]) * 1e3 for e in evs]
    step_steps = [e[0].elapsed_time(e[4]) * 1e3 for e in evs]

    f_fwd, f_bwd = w.flops_fwd(), w.flops_bwd()
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = f_fwd / (per_kernel["fwd_kernel"] * 1e-3) / 1e12
    bwd_ms = per_kernel["bwd_pre_kernel"] + per_kernel[main_name] + per_kernel[dq_name]
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12

    # Dominant kernel and its roofline (bf16 MFMA bound: attention is a dense
    # contraction).  Algorithmic FLOPs per launch: the forward does its 2
    # products (f_fwd); the backward's 5 products are f_bwd, of which the main
    # kernel does 4 (S, dP, dV, dK) in the fixed-order modes and all 5 in
    # atomic mode.  A fixed-order dQ kernel's algorithmic share is the dQ
    # product (1 of 5); the recompute mode's S and dP are overhead, not
    # algorithmic work.
    algo_flops = {"fwd_kernel": f_fwd, main_name: f_bwd * (0.8 if det else 1.0),
                  dq_name: f_bwd * 0.2 if det else 0.0}
    dom = max(("fwd_kernel", main_name, dq_name), key=lambda n: per_kernel[n])
    achieved = algo_flops[dom] / (per_kernel[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(dom, det),
                "avg_launch_us": round(per_kernel[dom] * 1e3, 1)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q, K, V, dO)",
        "config": {"workload": "attention forward+backward, B2 Hq16 Hkv16 N8192 D128 causal",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "D": D, "causal": True,
                   "dq_accumulation": DQ_LABEL[det],
                   "flops_per_step": f_fwd + f_bwd, "input_sha256": input_sha},
        "roofline": roofline,
        "fwd": {"tflops": round(fwd_tf, 1), "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "us": round(per_kernel["fwd_kernel"] * 1e3, 1), "us_spread": spread(fwd_steps)},
        "bwd": {"tflops": round(bwd_tf, 1), "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "us": round(bwd_ms * 1e3, 1), "us_spread": spread(bwd_steps),
                "kernels_us": {n: round(per_kernel[n] * 1e3, 1)
                               for n in names[1:]}},
        "step_us_spread": spread(step_steps),
        "host_wall_ms_per_step": round(wall / args.steps * 1e3, 4),
    }
    # The other dQ modes, timed on the same inputs for comparison (whole
    # fa_bwd call).
    out["bwd_other_modes"] = []
    for odet in sorted(set(DQ_MODES.values()) - {det}):
        ows_bytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D, odet)
        ows = torch.empty(ows_bytes, dtype=torch.uint8, device=dev)

        def obwd():
            check(fa.fa_bwd(P["q"], P["k"], P["v"], P["o"], P["lse"], P["do"], P["dq"], P["dk"],
                            P["dv"], B, Hq, Hkv, N, D, 1, w.scale, ows.data_ptr(), ows_bytes, odet,
                            sh), "fa_bwd")

        for _ in range(2):
            obwd()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            obwd()
        e1.record(stream)
        torch.cuda.synchronize()
        o_ms = e0.elapsed_time(e1) / 5
        out["bwd_other_modes"].append({"dq_accumulation": DQ_LABEL[odet],
                                       "us": round(o_ms * 1e3, 1),
                                       "tflops": round(f_bwd / (o_ms * 1e-3) / 1e12, 1),
                                       "workspace_bytes": ows_bytes})
        del ows
    out["bwd"]["workspace_bytes"] = ws_bytes
    if not args.no_extras:
        log("forward choices: exp2 polynomial share, rescale-heavy inputs")
        out["fwd_choices"] = bench_fwd_choices(fa, torch, dev, stream, P, w)
        log("forward rescale rate on the headline inputs")
        out["fwd_choices"]["rescale_rate"] = rescale_report(torch, dev)
        out["extras"] = {"varlen_fwd": bench_varlen(fa, torch, dev, stream),
                         "varlen_bwd": bench_varlen_bwd(fa, torch, dev, stream),
                         "varlen_bwd_stored_ds": bench_varlen_bwd(fa, torch, dev, stream, det=1),
                         "grouped_fwd_bwd": bench_grouped(fa, torch, dev, stream),
                         "decode_splitkv": bench_decode(fa, torch, dev, stream),
                         "fp8_fwd": bench_fp8(fa, torch, dev, stream, P, w),
                         "other_configs": bench_other_configs(fa, torch, dev, stream)}
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_heads} heads")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
