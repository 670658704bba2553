#!/usr/bin/env python3
"""Benchmark of the GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--procs 3] [--all]
    python bench.py --procs 1 --steps 5 --warmup 2 --no-cpu-baseline --calibration-copy
        (one in-process run: what rocprofv3 profiles, --pmc runs included)
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR SQ_DIR
        (turns those three rocprofv3 --pmc outputs into the committed summaries)

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill: LLaMA-3-8B-shaped causal prefill, bf16 in / fp32 accumulate,
    B=1 Hq=32 Hkv=8 N=2048 d=128 (gqa_attn_fwd), and
  * decode:  KV-cache decode, bf16 cache, B=8 Hq=12 Hkv=2 d=128, lengths
    U[512, 2048] (gqa_attn_decode: part kernel + merge kernel).
Both are checked against the CPU oracle before anything is timed.

Protocol (the same measurement repeated in --procs fresh child processes,
3 by default; the parent never touches the GPU and reports the median):
  * every configuration is parity-checked against the oracle, every element,
    in the process that times it;
  * the step loop: W untimed warm-up steps, then exactly K steps, each
    launch between HIP events of its own on the launch stream -- `value` is
    prefill TFLOP/s (algorithmic FLOPs = 4 * B * Hq * d * visible (query,
    key) pairs) over the prefill launch's average duration; the decode part
    is reported beside it in GB/s of algorithmic bytes (the K/V rows each
    sequence needs, plus q, o and the lengths), each decode call reading a
    different one of 48 independently drawn caches (768 MiB > the 256 MB
    Infinity Cache) so the reads come from HBM;
  * `configs`: each of the five named workloads timed on its own, 3 warm-ups
    then 5 windows of back-to-back calls of at least 10 ms each (a spin
    kernel queued ahead, so the host's issue time is not in the window),
    median and minimum per call;
  * `measured_peaks`: what this GPU sustains -- dense bf16 MFMA, streaming
    HBM read, the shader clock under MFMA load -- from libgqa_microbench.so.

`roofline` is for the prefill kernel (the dominant kernel of a step): bf16
dense MFMA peak 2500 TFLOP/s.  `traffic` (prefill and decode) comes from the
committed rocprofv3 counter summaries when they were taken from the current
kernel sources, else null.  `cpu_baseline` times the fp64 oracle on the
host, on the whole LLaMA prefill workload, in the first process only.

Only one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_FILE = os.path.join(PROFILES, "prefill_llama3_8b_counters.json")
DECODE_COUNTERS_FILE = os.path.join(PROFILES, "decode_b8_counters.json")
KERNEL_SOURCES = ["attn_tile.hpp", "prefill_kernel.hpp", "decode_kernel.hpp", "decode_part.hpp",
                  "mixed_kernel.hpp", "backward_kernel.hpp", "gqa_attn.hip"]
DECODE_SETS = 48  # 48 x 16 MiB of caches > 256 MB Infinity Cache
COPY_BYTES = 256 * 1024 * 1024  # calibration copy: reads and writes this many bytes
CHILD_TAG = "BENCH_CHILD_RESULT "


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mqa_flashattention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_flops(s) -> float:
    """4 FLOPs per (query, key, d) visible triple: QK^T and PV, 2 FLOPs per MAC."""
    return 4.0 * s.B * s.Hq * s.d * s.visible_pairs_per_head()


def decode_bytes(s, lens) -> float:
    """K and V rows each row needs, plus q, o and the lengths."""
    elem = 2 if str(s.dtype).endswith("bfloat16") else 4
    kv = float(sum(int(n) for n in lens)) * s.Hkv * s.d * 2 * elem
    return kv + 2.0 * s.B * s.Hq * s.d * elem + 4.0 * s.B


def append_bytes(s, positions) -> float:
    """Decode bytes over positions + 1 slots, plus the new K/V rows read and stored."""
    elem = 2 if str(s.dtype).endswith("bfloat16") else 4
    lens = [int(p) + 1 for p in positions if 0 <= int(p) < s.Smax]
    return decode_bytes(s, lens) + 4.0 * len(lens) * s.Hkv * s.d * elem


def fwd_bytes(s) -> float:
    elem = 2 if str(s.dtype).endswith("bfloat16") else 4
    return elem * (2.0 * s.B * s.Hq * s.Nq * s.d + 2.0 * s.B * s.Hkv * s.Nk * s.d)


def traffic_from_counters(path=COUNTERS_FILE):
    """Measured HBM bytes per launch from a committed counter summary, if it
    was taken from the current kernel sources."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def check(out, ref, tol, what):
    import numpy as np
    err = float(np.max(np.abs(out.detach().cpu().double().numpy() - ref)))
    if not err <= tol:
        raise SystemExit(f"{what}: parity check failed, max abs error {err} > {tol}")
    return err


def head_start(steps):
    """Queue a spin kernel of about 5 ms + 50 us per call on the current stream.

    The host needs longer to issue one decode call (Python argument checks,
    event records) than the call takes on the GPU; without a head start the
    GPU catches up and idles, and an event pair around a call then also
    counts the host time spent issuing it."""
    import torch
    torch.cuda._sleep(int(2.4e9 * (5e-3 + 50e-6 * steps)))


def time_fwd_workload(s, steps, warmup, bthd=False):
    """Event-timed average duration (ms) of one gqa_attn_fwd launch; with bthd,
    of one gqa_attn_fwd_strided launch on token-major [B, N, H, d] tensors."""
    import torch
    from mqa_flashattention_amd import attn_fwd, attn_fwd_strided
    from mqa_flashattention_amd.workloads import fwd_inputs
    q, k, v = (t.cuda() for t in fwd_inputs(s, 0))
    fn = attn_fwd
    if bthd:
        q, k, v = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
        fn = attn_fwd_strided
    out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    for _ in range(warmup):
        fn(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_persistent_causal(steps, warmup):
    """The LLaMA-3-8B causal prefill layer at batch 4: 2048 units of 128
    columns, more than two per resident workgroup, so the launch runs on the
    persistent schedule (per-XCD atomic queues, heaviest position blocks
    first, stealing).  A sample of rows is checked against the oracle first.
    Returns (shape, event-timed average duration in ms)."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import attn_fwd
    from mqa_flashattention_amd.workloads import WORKLOADS, FwdShape, fwd_inputs
    ps = WORKLOADS["llama3_8b_prefill"].fwd[0]
    s = FwdShape(4, ps.Hq, ps.Hkv, ps.Nq, ps.Nk, ps.d, True, 0, ps.dtype)
    host = fwd_inputs(s, 0)
    q, k, v = (t.cuda() for t in host)
    out = attn_fwd(q, k, v, causal=True, scale=s.scale)
    torch.cuda.synchronize()
    n = s.B * s.Hq * s.Nq
    ids = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(6).integers(0, n, 62)]))
    ref = oracle.attn_fwd_rows(host[0], host[1], host[2], ids, causal=True, scale=s.scale)
    check(out.reshape(-1, s.d)[torch.from_numpy(ids).cuda()], ref, 2e-2,
          "batch-4 LLaMA prefill (persistent schedule)")
    for _ in range(warmup):
        attn_fwd(q, k, v, causal=True, scale=s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        attn_fwd(q, k, v, causal=True, scale=s.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    return s, e0.elapsed_time(e1) / steps


def time_append_workload(s, steps, warmup):
    """Event-timed average duration (ms) of one gqa_attn_decode_append call,
    each call on a different one of DECODE_SETS cache pairs (HBM-cold), after
    a parity check of the first call against the oracle (outputs and caches)."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import attn_decode_append, decode_workspace_bytes
    from mqa_flashattention_amd.workloads import append_inputs
    dev = torch.device("cuda:0")
    q_h, kn_h, vn_h, kc_h, vc_h, pos_h = append_inputs(s, 0)
    q, kn, vn, pos = q_h.to(dev), kn_h.to(dev), vn_h.to(dev), pos_h.to(dev)
    kcs, vcs = [kc_h.to(dev)], [vc_h.to(dev)]
    gen = torch.Generator(device=dev).manual_seed(2)
    for _ in range(DECODE_SETS - 1):
        kcs.append(torch.randn(kc_h.shape, generator=gen, device=dev).to(s.dtype))
        vcs.append(torch.randn(vc_h.shape, generator=gen, device=dev).to(s.dtype))
    o = torch.empty_like(q)
    ws = torch.empty(decode_workspace_bytes(s.B, s.Hq, s.Hkv, s.Smax, s.d), dtype=torch.uint8,
                     device=dev)
    attn_decode_append(q, kn, vn, kcs[0], vcs[0], pos, scale=s.scale, out=o, workspace=ws)
    torch.cuda.synchronize()
    ref, kref, vref = oracle.attn_decode_append(q_h, kn_h, vn_h, kc_h, vc_h, pos_h, scale=s.scale)
    check(o, ref, 2e-2, "decode_append")
    if not (np.array_equal(kcs[0].cpu().double().numpy(), kref)
            and np.array_equal(vcs[0].cpu().double().numpy(), vref)):
        raise SystemExit("decode_append: updated caches differ from the oracle")
    for i in range(warmup):
        attn_decode_append(q, kn, vn, kcs[i % DECODE_SETS], vcs[i % DECODE_SETS], pos,
                           scale=s.scale, out=o, workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    head_start(steps)
    for i in range(steps):
        ev[i][0].record()
        attn_decode_append(q, kn, vn, kcs[(i + 1) % DECODE_SETS], vcs[(i + 1) % DECODE_SETS],
                           pos, scale=s.scale, out=o, workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])), pos_h.tolist()


def time_decode_graph(steps):
    """Decode of the batch-8 workload replayed from a HIP graph: one graph of
    DECODE_SETS calls (one per HBM-cold cache set, caller-provided
    workspace), replayed `steps` times; returns ms per call.  Before timing,
    the graph's last call is checked bit for bit against the same call made
    eagerly, after a first replay and again after the timed ones."""
    import numpy as np
    import torch
    from mqa_flashattention_amd import attn_decode, decode_workspace_bytes
    from mqa_flashattention_amd.workloads import WORKLOADS, decode_inputs
    s = WORKLOADS["kv_decode_b8"].decode
    dev = torch.device("cuda:0")
    q_h, k_h, v_h, l_h = decode_inputs(s, 0)
    q, lens = q_h.to(dev), l_h.to(dev)
    kcs, vcs = [k_h.to(dev)], [v_h.to(dev)]
    gen = torch.Generator(device=dev).manual_seed(3)
    for _ in range(DECODE_SETS - 1):
        kcs.append(torch.randn(k_h.shape, generator=gen, device=dev).to(s.dtype))
        vcs.append(torch.randn(v_h.shape, generator=gen, device=dev).to(s.dtype))
    ws = torch.empty(decode_workspace_bytes(s.B, s.Hq, s.Hkv, s.Smax, s.d), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    want = attn_decode(q, kcs[-1], vcs[-1], lens, scale=s.scale, workspace=ws).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(DECODE_SETS):
            attn_decode(q, kcs[i], vcs[i], lens, scale=s.scale, out=o, workspace=ws)
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(o, want):
        raise SystemExit("decode graph replay differs from the eager call")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        graph.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    if not torch.equal(o, want):
        raise SystemExit("decode graph replay differs from the eager call")
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev])) / DECODE_SETS
    return ms, decode_bytes(s, l_h.tolist())


def varlen_flops(lens, Hq, d) -> float:
    """Causal whole prompts: 4 * Hq * d per visible (query, key) pair."""
    return sum(4.0 * Hq * d * L * (L + 1) / 2 for L in lens)


def time_varlen_workload(steps, warmup):
    """The mixed-length prompt batch through one gqa_attn_fwd_varlen launch,
    checked in full against the oracle, and the same prompts as one
    gqa_attn_fwd call each: event-timed ms per batch, both ways."""
    import numpy as np
    import torch
    import oracle
    from mqa_flashattention_amd import attn_fwd, attn_fwd_varlen
    from mqa_flashattention_amd.workloads import VARLEN_PREFILL as s, varlen_inputs, varlen_lengths
    lens = varlen_lengths(s)
    qh, kh, vh, cqh, ckh = varlen_inputs(lens, lens, s.Hq, s.Hkv, s.d, s.dtype, 0)
    q, k, v, cq, ck = (t.cuda() for t in (qh, kh, vh, cqh, ckh))
    out = torch.empty_like(q)
    attn_fwd_varlen(q, k, v, cq, ck, max(lens), causal=True, out=out)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd_varlen(qh, kh, vh, cqh, ckh, causal=True)
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    if not err <= 2e-2:
        raise SystemExit(f"parity failure (varlen prompt batch): max abs error {err}")
    # per-prompt [1, H, L, d] copies for the one-call-per-prompt comparison
    per = []
    for i, L in enumerate(lens):
        a, b = int(cqh[i]), int(cqh[i + 1])
        per.append(tuple(t[a:b].transpose(0, 1)[None].contiguous().cuda() for t in (qh, kh, vh)))
    outs = [torch.empty_like(p[0]) for p in per]

    def packed():
        attn_fwd_varlen(q, k, v, cq, ck, max(lens), causal=True, out=out)

    def separate():
        for (a, b, c), o in zip(per, outs):
            attn_fwd(a, b, c, causal=True, out=o)

    res = []
    for fn in (packed, separate):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        head_start(steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / steps)
    return res[0], res[1], lens, err


def bwd_flops(s) -> float:
    """Algorithmic backward FLOPs: five contractions over the visible pairs
    (S recomputed, dP, dV, dK, dQ), 2 FLOPs per MAC -- 2.5x the forward."""
    return 10.0 * s.B * s.Hq * s.d * s.visible_pairs_per_head()


def time_bwd_workload(s, steps, warmup):
    """Event-timed average duration (ms) of one gqa_attn_bwd call (both of its
    kernels), after a parity check of dQ, dK, dV against the oracle."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import attn_bwd, attn_fwd, bwd_workspace_bytes
    from mqa_flashattention_amd.workloads import fwd_inputs, random_tensor
    q_h, k_h, v_h = fwd_inputs(s, 0)
    do_h = random_tensor(q_h.shape, 11, s.dtype)
    q, k, v, do = (t.cuda() for t in (q_h, k_h, v_h, do_h))
    o = attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    ws = torch.empty(bwd_workspace_bytes(s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.d), dtype=torch.uint8,
                     device=q.device)
    grads = attn_bwd(q, k, v, o, do, causal=s.causal, q_offset=s.q_offset, scale=s.scale,
                     workspace=ws)
    torch.cuda.synchronize()
    want = oracle.attn_bwd(q_h, k_h, v_h, do_h, causal=s.causal, q_offset=s.q_offset,
                           scale=s.scale)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        got = g.detach().cpu().double().numpy()
        if not np.all(np.abs(got - w) <= 2e-2 + 2.0 ** -7 * np.abs(w)):
            raise SystemExit(f"backward {name}: parity check failed")
    for _ in range(warmup):
        attn_bwd(q, k, v, o, do, causal=s.causal, q_offset=s.q_offset, scale=s.scale,
                 workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        attn_bwd(q, k, v, o, do, causal=s.causal, q_offset=s.q_offset, scale=s.scale,
                 workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def time_mixed_workload(w, steps, warmup, sets=3):
    """Event-timed average duration (ms) of one gqa_attn_mixed call (the
    persistent launch and the decode combine), and of the same work as two
    calls (gqa_attn_fwd on the chunk, then gqa_attn_decode), after a parity
    check of both outputs against the oracle.  The decode caches cycle over
    `sets` copies (more bytes than the Infinity Cache holds), so each call
    reads them from HBM as a serving step would."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import (attn_decode, attn_fwd, attn_mixed,
                                        decode_workspace_bytes)
    from mqa_flashattention_amd.workloads import mixed_inputs
    c, r = w.fwd[0], w.decode
    host = mixed_inputs(c, r, 0)
    q, k, v = (t.cuda() for t in host[:3])
    qd, sl = host[3].cuda(), host[6].cuda()
    caches = [(host[4].cuda(), host[5].cuda())]
    caches += [(torch.roll(caches[0][0], i, 2).contiguous(), torch.roll(caches[0][1], i, 2).contiguous())
               for i in range(1, sets)]
    ws = torch.empty(decode_workspace_bytes(r.B, r.Hq, r.Hkv, r.Smax, r.d), dtype=torch.uint8,
                     device=q.device)
    o, od = attn_mixed(q, k, v, c.q_offset, qd, *caches[0], sl, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    ids = np.unique(np.random.default_rng(5).integers(0, c.B * c.Hq * c.Nq, 64))
    ref = oracle.attn_fwd_rows(host[0], host[1], host[2], ids, causal=True, q_offset=c.q_offset,
                               scale=c.scale)
    check(o.reshape(-1, c.d)[torch.from_numpy(ids).cuda()], ref, 2e-2, "mixed batch chunk")
    check(od, oracle.attn_decode(host[3], host[4], host[5], host[6], scale=c.scale), 2e-2,
          "mixed batch decode rows")

    def mixed(i):
        attn_mixed(q, k, v, c.q_offset, qd, *caches[i % sets], sl, scale=c.scale, out=o,
                   out_decode=od, workspace=ws)

    def separate(i):
        attn_fwd(q, k, v, causal=True, q_offset=c.q_offset, scale=c.scale, out=o)
        attn_decode(qd, *caches[i % sets], sl, scale=c.scale, out=od, workspace=ws)

    res = []
    for fn in (mixed, separate):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        res.append(float(np.mean([a.elapsed_time(b) for a, b in ev])))
    return res[0], res[1], sl


# Supplementary decode sweep: the batch-8 shape (Hq 12, Hkv 2, d 128) at more
# rows and longer contexts, lengths uniform in [Smax/4, Smax] as for the
# batch-8 workload's [512, 2048].  It shows how close the decode kernels come
# to HBM bandwidth once a call moves enough bytes to hide launch and latency.
DECODE_SWEEP = [(b, smax) for smax in (2048, 8192) for b in (8, 32, 128)]
SWEEP_COLD_BYTES = 768 * 1024 * 1024  # caches cycled per sweep point (> Infinity Cache)


def time_decode_sweep(steps, warmup):
    """Event-timed decode calls at each DECODE_SWEEP point, HBM-cold caches.

    Inputs are N(0,1) bf16 drawn on the GPU from a seeded generator, lengths
    from a seeded CPU generator.  Before timing, rows 0 and B-1 of the first
    call are checked against the oracle."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import attn_decode, decode_workspace_bytes
    from mqa_flashattention_amd.workloads import DecodeShape

    dev = torch.device("cuda:0")
    out = {}
    for B, smax in DECODE_SWEEP:
        s = DecodeShape(B, 12, 2, smax, 128, smax // 4, smax)
        gen = torch.Generator(device=dev).manual_seed(100 + B + smax)
        lens_h = torch.randint(s.len_lo, s.len_hi + 1, (B,),
                               generator=torch.Generator().manual_seed(B + smax),
                               dtype=torch.int64).to(torch.int32)
        lens = lens_h.to(dev)
        q = torch.randn((B, s.Hq, s.d), generator=gen, device=dev).to(torch.bfloat16)
        shape = (B, s.Hkv, smax, s.d)
        set_bytes = 2 * B * s.Hkv * smax * s.d * 2
        nsets = max(2, -(-SWEEP_COLD_BYTES // set_bytes))
        kcs = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
               for _ in range(nsets)]
        vcs = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
               for _ in range(nsets)]
        o = torch.empty_like(q)
        ws = torch.empty(decode_workspace_bytes(B, s.Hq, s.Hkv, smax, s.d), dtype=torch.uint8,
                         device=dev)
        attn_decode(q, kcs[0], vcs[0], lens, scale=s.scale, out=o, workspace=ws)
        torch.cuda.synchronize()
        for r in sorted({0, B - 1}):
            ref = oracle.attn_decode(q[r:r + 1].cpu(), kcs[0][r:r + 1].cpu(),
                                     vcs[0][r:r + 1].cpu(), lens_h[r:r + 1], scale=s.scale)
            check(o[r:r + 1], ref, 2e-2, f"decode sweep B{B} Smax{smax} row {r}")
        for i in range(warmup):
            attn_decode(q, kcs[i % nsets], vcs[i % nsets], lens, scale=s.scale, out=o,
                        workspace=ws)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        head_start(steps)
        for i in range(steps):
            ev[i][0].record()
            attn_decode(q, kcs[(i + 1) % nsets], vcs[(i + 1) % nsets], lens, scale=s.scale,
                        out=o, workspace=ws)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        nbytes = decode_bytes(s, lens_h.tolist())
        gb = nbytes / (ms * 1e-3) / 1e9
        out[f"decode_sweep[B={B},Smax={smax}]"] = {
            "ms": round(ms, 5), "value": round(gb, 1), "unit": "GB/s",
            "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
            "algorithmic_mb": round(nbytes / 1e6, 3), "cache_sets": nsets}
        del kcs, vcs, q, o, ws
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- machine peaks

def measured_peaks():
    """Dense bf16 MFMA rate, streaming HBM read rate and the shader clock under
    MFMA load on this GPU (libgqa_microbench.so), each the best of 5 timed
    launches after a warm-up."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mqa_flashattention_amd", "libgqa_microbench.so"))
    lib.gqa_mb_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.gqa_mb_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = cus * 2, 4096                  # 8 waves per CU, two per SIMD
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device=dev)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return min(out)

    def mfma():
        if lib.gqa_mb_mfma_bf16(blocks, iters, ctypes.c_void_p(clk.data_ptr()),
                                ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise SystemExit("MFMA microbenchmark launch failed")

    t = best(mfma)
    flops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 16
    ticks, ref = clk.tolist()
    nbytes = 2 << 30                                 # 2 GiB > 256 MB Infinity Cache
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    rsink = torch.zeros(256, dtype=torch.int32, device=dev)

    def read():
        if lib.gqa_mb_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(rsink.data_ptr()),
                           cus * 16, stream) != 0:
            raise SystemExit("read microbenchmark launch failed")

    tr = best(read)
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flops / t / 1e12, 1),
            "hbm_read_gbps": round(nbytes / tr / 1e9, 1),
            "sclk_ghz_under_mfma": round(ticks / (ref / 100e6) / 1e9, 3) if ref else None,
            "note": "libgqa_microbench.so: 32x32x16 bf16 MFMA stream in registers (8 waves "
                    "per CU); 16-byte non-temporal streaming read of 2 GiB (16 waves per CU, "
                    "8 loads in flight each); wave 0's s_memtime over s_memrealtime (100 MHz) "
                    "across the MFMA kernel"}


LDS_PATTERNS = [
    # (pattern id of gqa_mb_lds, access, what it is)
    (0, "16-byte read", "linear (lane * 16)"),
    (1, "16-byte read", "forward K fragments: k_row_perm rows of 272 bytes"),
    (2, "16-byte read", "forward V^T fragments: 32 consecutive 80-byte rows"),
    (3, "16-byte read", "dK/dV score operands: rows 8 (n/4) + 4 qb + n%4 of 272 bytes"),
    (4, "16-byte read", "dK/dV transposed operands: 16 consecutive 80-byte rows"),
    (5, "16-byte read", "case 3 from 256-byte rows, row 16 qb + n, chunk XOR row"),
    (6, "16-byte read", "case 4 from 96-byte rows"),
    (7, "4-byte write", "linear (lane * 4)"),
    (8, "4-byte write", "transposed staging: two-key words into 80-byte rows"),
    (9, "16-byte write", "linear (lane * 16)"),
    (10, "16-byte write", "row-major staging: rows 2n + i of 272 bytes"),
]


def lds_probe():
    """Time every LDS access pattern of gqa_mb_lds (libgqa_microbench.so): 4 waves
    per block, one block per CU, each wave repeating its pattern 4096 x 16
    times; best of 5 launches after a warm-up.  The ratio to the linear
    pattern of the same access width is the pattern's bank-conflict factor."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mqa_flashattention_amd", "libgqa_microbench.so"))
    lib.gqa_mb_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    reps = 4096
    rows, base = [], {}
    for pat, access, what in LDS_PATTERNS:
        def run():
            if lib.gqa_mb_lds(pat, cus, reps, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise SystemExit("LDS microbenchmark launch failed")
        run()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = min(times)
        base.setdefault(access, ms)
        rows.append({"pattern": pat, "access": access, "what": what, "ms": round(ms, 4),
                     "ns_per_wave_instruction": round(ms * 1e6 / (reps * 16 * 4), 3),
                     "vs_linear": round(ms / base[access], 2)})
    return rows


def valu_probe():
    """fp32 FMA and exp2 rates (libgqa_microbench.so gqa_mb_valu): eight
    independent chains per lane, 8 waves per CU; lane operations per clock
    per CU from the kernel time and wave 0's clock counters (best of 5), at 8
    and at 16 waves per CU."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mqa_flashattention_amd", "libgqa_microbench.so"))
    lib.gqa_mb_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    sink = torch.zeros(cus * 4 * 256, dtype=torch.float32, device=dev)
    out = []
    cases = [(op, name, iters, wpc) for wpc in (8, 16)
             for op, name, iters in ((0, "fp32 FMA (v_fma_f32)", 1 << 16),
                                     (1, "exp2 (v_exp_f32, plus a subtraction)", 1 << 14))]
    for op, name, iters, wpc in cases:
        blocks = cus * wpc // 4
        def run():
            if lib.gqa_mb_valu(op, blocks, iters, ctypes.c_void_p(clk.data_ptr()),
                               ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise SystemExit("VALU microbenchmark launch failed")
        run()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            if best is None or t < best[0]:
                best = (t, clk.tolist())
        t, (ticks, ref) = best
        ghz = ticks / (ref / 100e6) / 1e9 if ref else None
        lane_ops = blocks * 256 * iters * 8
        out.append({"op": name, "waves_per_cu": wpc, "ms": round(t * 1e3, 3),
                    "sclk_ghz": round(ghz, 3) if ghz else None,
                    "lane_ops_per_clk_per_cu": round(lane_ops / t / (ghz * 1e9) / cus, 1) if ghz else None})
    return out


# ---------------------------------------------------------------- per-config windows# ---------------------------------------------------------------- per-config windows

def time_windows(fn, nwin=5, min_ms=10.0):
    """Per-call duration of fn (one launch on the current stream): 3 warm-up
    calls, then nwin windows of R back-to-back calls between two events, R
    chosen so a window lasts >= min_ms; a spin kernel queued ahead of each
    window keeps the host's issue time out of it.  Returns (median, min) ms."""
    import numpy as np
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    head_start(20)
    e0.record()
    for i in range(20):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 20, 1e-4)
    reps = int(min(5000, max(20, math.ceil(min_ms / per))))
    out = []
    for _ in range(nwin):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        head_start(reps)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    return float(np.median(out)), float(min(out)), reps


def measure_configs(peaks, windows=True):
    """Every named workload: full oracle parity, then windowed timing (or,
    without windows, three more calls each: what a counter run profiles)."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate only
    from mqa_flashattention_amd import attn_decode, attn_fwd, decode_workspace_bytes
    from mqa_flashattention_amd.workloads import WORKLOADS, decode_inputs, fwd_inputs
    dev = torch.device("cuda:0")
    out = {}
    fwd = [("c0 tiny_gqa_f32", WORKLOADS["tiny_gqa_f32"].fwd[0]),
           ("c1 llama3_8b_prefill", WORKLOADS["llama3_8b_prefill"].fwd[0])]
    fwd += [(f"c2 mha_gqa_mqa_sweep[Hkv={s.Hkv}]", s) for s in WORKLOADS["mha_gqa_mqa_sweep"].fwd]
    fwd += [("c4 chunked_prefill_4k", WORKLOADS["chunked_prefill_4k"].fwd[0])]
    for name, s in fwd:
        q_h, k_h, v_h = fwd_inputs(s, 0)
        q, k, v = q_h.to(dev), k_h.to(dev), v_h.to(dev)
        o = torch.empty_like(q)

        def call(i, q=q, k=k, v=v, o=o, s=s):
            attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale, out=o)

        call(0)
        torch.cuda.synchronize()
        ref = oracle.attn_fwd(q_h, k_h, v_h, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
        tol = 1e-4 if s.dtype == torch.float32 else 2e-2
        err = check(o, ref, tol, name)
        if not windows:
            for i in range(3):
                call(i)
            torch.cuda.synchronize()
            out[name] = {"parity_max_abs_err": float(f"{err:.3e}")}
            continue
        med, mn, reps = time_windows(call)
        tf = prefill_flops(s) / (med * 1e-3) / 1e12
        f32 = s.dtype == torch.float32
        entry = {"ms_median": round(med, 5), "ms_min": round(mn, 5), "calls_per_window": reps,
                 "tflops": round(tf, 2), "parity_max_abs_err": float(f"{err:.3e}"),
                 "shape": f"B{s.B} Hq{s.Hq} Hkv{s.Hkv} Nq{s.Nq} Nk{s.Nk} d{s.d} "
                          f"{'causal@' + str(s.q_offset) if s.causal else 'non-causal'} "
                          f"{'fp32' if f32 else 'bf16'}"}
        if f32:
            entry["note"] = "correctness workload: no roofline claim"
        else:
            entry["frac_mfma_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            if peaks and peaks.get("mfma_bf16_tflops"):
                entry["frac_measured_mfma_peak"] = round(tf / peaks["mfma_bf16_tflops"], 4)
        out[name] = entry
        del q, k, v, o
    # c3: the batch-8 decode, HBM-cold caches
    ds = WORKLOADS["kv_decode_b8"].decode
    dq_h, dk_h, dv_h, dl_h = decode_inputs(ds, 0)
    dq, dl = dq_h.to(dev), dl_h.to(dev)
    kcs, vcs = [dk_h.to(dev)], [dv_h.to(dev)]
    gen = torch.Generator(device=dev).manual_seed(1)
    for _ in range(DECODE_SETS - 1):
        kcs.append(torch.randn(dk_h.shape, generator=gen, device=dev).to(ds.dtype))
        vcs.append(torch.randn(dv_h.shape, generator=gen, device=dev).to(ds.dtype))
    do = torch.empty_like(dq)
    ws = torch.empty(decode_workspace_bytes(ds.B, ds.Hq, ds.Hkv, ds.Smax, ds.d),
                     dtype=torch.uint8, device=dev)

    def dcall(i):
        attn_decode(dq, kcs[i % DECODE_SETS], vcs[i % DECODE_SETS], dl, scale=ds.scale, out=do,
                    workspace=ws)

    dcall(0)
    torch.cuda.synchronize()
    err = check(do, oracle.attn_decode(dq_h, dk_h, dv_h, dl_h, scale=ds.scale), 2e-2, "c3 decode")
    if not windows:
        for i in range(3):
            dcall(i + 1)
        torch.cuda.synchronize()
        out["c3 kv_decode_b8"] = {"parity_max_abs_err": float(f"{err:.3e}")}
        return out
    med, mn, reps = time_windows(dcall)
    nbytes = decode_bytes(ds, dl_h.tolist())
    gb = nbytes / (med * 1e-3) / 1e9
    entry = {"ms_median": round(med, 5), "ms_min": round(mn, 5), "calls_per_window": reps,
             "gbps": round(gb, 1), "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
             "algorithmic_mb": round(nbytes / 1e6, 4), "parity_max_abs_err": float(f"{err:.3e}"),
             "shape": f"B{ds.B} Hq{ds.Hq} Hkv{ds.Hkv} Smax{ds.Smax} d{ds.d} bf16, "
                      f"sum(lengths)={int(dl_h.sum())}, {DECODE_SETS} cache sets cycled"}
    if peaks and peaks.get("hbm_read_gbps"):
        entry["frac_measured_hbm_read"] = round(gb / peaks["hbm_read_gbps"], 4)
    out["c3 kv_decode_b8"] = entry
    del kcs, vcs
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- one process

def run_child(args):
    """The whole measurement in this process; returns the result dict."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: parity gate and CPU baseline only
    from mqa_flashattention_amd import attn_decode, attn_fwd, decode_workspace_bytes
    from mqa_flashattention_amd.workloads import WORKLOADS, decode_inputs, fwd_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ps = WORKLOADS["llama3_8b_prefill"].fwd[0]
    ds = WORKLOADS["kv_decode_b8"].decode

    # ---------------- inputs (seed 0, resident in HBM before timing)
    q_h, k_h, v_h = fwd_inputs(ps, 0)
    q, k, v = q_h.to(dev), k_h.to(dev), v_h.to(dev)
    o = torch.empty_like(q)
    dq_h, dk_h, dv_h, dl_h = decode_inputs(ds, 0)
    dq, dl = dq_h.to(dev), dl_h.to(dev)
    kcs, vcs = [dk_h.to(dev)], [dv_h.to(dev)]
    gen = torch.Generator(device=dev).manual_seed(1)
    for _ in range(DECODE_SETS - 1):
        kcs.append(torch.randn(dk_h.shape, generator=gen, device=dev).to(ds.dtype))
        vcs.append(torch.randn(dv_h.shape, generator=gen, device=dev).to(ds.dtype))
    do = torch.empty_like(dq)
    ws = torch.empty(decode_workspace_bytes(ds.B, ds.Hq, ds.Hkv, ds.Smax, ds.d),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        attn_fwd(q, k, v, causal=True, scale=ps.scale, out=o)

    def decode(i):
        attn_decode(dq, kcs[i], vcs[i], dl, scale=ds.scale, out=do, workspace=ws)

    # ---------------- parity gate (before any timing)
    prefill()
    decode(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ref = oracle.attn_fwd(q_h, k_h, v_h, causal=True, scale=ps.scale)
    oracle_s = time.perf_counter() - t0
    prefill_err = check(o, ref, 2e-2, "prefill")
    t0 = time.perf_counter()
    dref = oracle.attn_decode(dq_h, dk_h, dv_h, dl_h, scale=ds.scale)
    oracle_dec_s = time.perf_counter() - t0
    decode_err = check(do, dref, 2e-2, "decode")
    print(f"# parity ok: prefill max err {prefill_err:.2e}, decode max err {decode_err:.2e}",
          file=sys.stderr, flush=True)

    # ---------------- warmup + timed steps
    for i in range(args.warmup):
        prefill()
        decode(i % DECODE_SETS)
    torch.cuda.synchronize()
    # Each launch between an event pair of its own, steps interleaved as a
    # serving loop would issue them; the host issues a step faster than the
    # GPU runs it, so the pairs bracket GPU work only.
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        decode(i % DECODE_SETS)
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / K
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    del kcs, vcs
    torch.cuda.empty_cache()

    flops = prefill_flops(ps)
    lens = dl_h.tolist()
    dbytes = decode_bytes(ds, lens)
    res = {"prefill_ms": pre_ms, "decode_ms": dec_ms, "ms_per_step": ms_per_step,
           "wall_s_timed": wall, "prefill_tflops": flops / (pre_ms * 1e-3) / 1e12,
           "decode_gbps": dbytes / (dec_ms * 1e-3) / 1e9}

    if args.calibration_copy:
        # a plain streaming kernel of known traffic: reads and writes COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.counters_run:
        # what the rocprofv3 --pmc runs collect: every config's kernels a few
        # times, the calibration copy and the MFMA microbenchmark
        measured_peaks()
        measure_configs(None, windows=False)
        return None
    res["peaks"] = measured_peaks()
    res["configs"] = measure_configs(res["peaks"])
    if args.cpu_baseline:
        res["cpu_baseline"] = {
            "value": round(flops / oracle_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole prefill workload (B1 Hq32 Hkv8 N2048 d128 causal), fp64, "
                      f"{oracle_s:.2f} s wall",
            "decode_gbps": round(dbytes / oracle_dec_s / 1e9, 4),
        }
    if args.all:
        res["other_workloads"] = other_workloads(K)
    return res


def other_workloads(K):
    from mqa_flashattention_amd.workloads import WORKLOADS
    ps = WORKLOADS["llama3_8b_prefill"].fwd[0]
    extra = {}
    ms = time_fwd_workload(ps, max(10, K // 2), 3, bthd=True)
    tf = prefill_flops(ps) / (ms * 1e-3) / 1e12
    extra["llama3_8b_prefill[bthd]"] = {
        "ms": round(ms, 5), "tflops": round(tf, 2),
        "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "token-major [B, N, H, d] Q/K/V/O through gqa_attn_fwd_strided, no copies"}
    s4, ms = time_persistent_causal(max(10, K // 4), 3)
    tf = prefill_flops(s4) / (ms * 1e-3) / 1e12
    extra["llama3_8b_prefill_b4[persistent]"] = {
        "ms": round(ms, 5), "tflops": round(tf, 2),
        "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "the LLaMA-3-8B causal layer at batch 4 (2048 128-column units): the "
                "persistent schedule's per-XCD atomic queues, heaviest first, with stealing; "
                "sampled rows checked against the oracle"}
    sa = WORKLOADS["kv_decode_append_b8"].decode
    ms, positions = time_append_workload(sa, max(20, K), 5)
    gb = append_bytes(sa, positions) / (ms * 1e-3) / 1e9
    extra["kv_decode_append_b8"] = {
        "ms": round(ms, 5), "value": round(gb, 2), "unit": "GB/s",
        "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
        "algorithmic_mb": round(append_bytes(sa, positions) / 1e6, 4),
        "note": "store of the new K/V rows + attention + merge, one call, HBM-cold caches"}
    ms, nbytes = time_decode_graph(20)
    gb = nbytes / (ms * 1e-3) / 1e9
    extra["kv_decode_b8[graph]"] = {
        "ms": round(ms, 5), "value": round(gb, 2), "unit": "GB/s",
        "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
        "note": "the same decode calls replayed from a HIP graph (48 per replay, one per "
                "HBM-cold cache set): no host dispatch between calls"}
    ms = time_bwd_workload(ps, max(10, K // 2), 3)
    tf = bwd_flops(ps) / (ms * 1e-3) / 1e12
    extra["llama3_8b_backward"] = {
        "ms": round(ms, 5), "tflops": round(tf, 2),
        "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "algorithmic_gflop": round(bwd_flops(ps) / 1e9, 4),
        "note": "gqa_attn_bwd: dQ kernel (one pass, online softmax, row statistics), "
                "dK/dV kernel (query range of each key block in up to 16 parts) and their "
                "merge; 5 contractions counted (the kernels execute 6: S twice)"}
    for name in ("llama3_8b_mixed", "llama3_8b_mixed_c128"):
        wm = WORKLOADS[name]
        ms, ms_sep, lens_m = time_mixed_workload(wm, max(20, K), 5)
        extra[name] = {
            "ms": round(ms, 5), "ms_as_two_calls": round(ms_sep, 5),
            "speedup_vs_two_calls": round(ms_sep / ms, 4),
            "chunk_gflop": round(prefill_flops(wm.fwd[0]) / 1e9, 4),
            "decode_mb": round(decode_bytes(wm.decode, lens_m) / 1e6, 4),
            "note": f"gqa_attn_mixed: the {wm.fwd[0].Nq}-query chunk and {wm.decode.B} decode "
                    "rows in one persistent launch + its merge launches (the chunk's cut "
                    "units when it runs on the balanced schedule, the decode rows), against "
                    "gqa_attn_fwd then gqa_attn_decode; decode caches HBM-cold"}
    ms, ms_sep, lens, err = time_varlen_workload(max(10, K // 2), 3)
    from mqa_flashattention_amd.workloads import VARLEN_PREFILL as vs
    tf = varlen_flops(lens, vs.Hq, vs.d) / (ms * 1e-3) / 1e12
    extra["varlen_prompt_batch"] = {
        "ms": round(ms, 5), "tflops": round(tf, 2),
        "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "ms_as_one_call_per_prompt": round(ms_sep, 5),
        "speedup_vs_one_call_per_prompt": round(ms_sep / ms, 4),
        "lengths": lens, "max_abs_err": err,
        "note": f"{vs.nseq} causal prompts of {vs.len_lo}..{vs.len_hi} tokens packed "
                f"token-major (Hq {vs.Hq}, Hkv {vs.Hkv}, d {vs.d}, bf16) in one "
                "gqa_attn_fwd_varlen launch, every element checked against the oracle"}
    extra.update(time_decode_sweep(20, 3))
    return extra


# ---------------------------------------------------------------- the report

def _median(xs):
    xs = [x for x in xs if x is not None]
    return statistics.median(xs) if xs else None


def report(children, args):
    """One JSON line from the child results: medians over the processes."""
    from mqa_flashattention_amd.workloads import WORKLOADS
    ps = WORKLOADS["llama3_8b_prefill"].fwd[0]
    ds = WORKLOADS["kv_decode_b8"].decode
    from mqa_flashattention_amd.workloads import decode_inputs
    lens = decode_inputs(ds, 0)[3].tolist()
    flops = prefill_flops(ps)
    dbytes = decode_bytes(ds, lens)
    pre_ms = _median([c["prefill_ms"] for c in children])
    dec_ms = _median([c["decode_ms"] for c in children])
    tflops = flops / (pre_ms * 1e-3) / 1e12
    gbps = dbytes / (dec_ms * 1e-3) / 1e9
    peaks = {k: _median([c["peaks"][k] for c in children])
             for k in ("mfma_bf16_tflops", "hbm_read_gbps", "sclk_ghz_under_mfma")}
    peaks["note"] = children[0]["peaks"]["note"]
    configs = {}
    for name in children[0]["configs"]:
        rows = [c["configs"][name] for c in children]
        e = dict(rows[0])
        for key in ("ms_median", "ms_min", "tflops", "gbps", "frac_mfma_peak",
                    "frac_measured_mfma_peak", "frac_hbm_peak", "frac_measured_hbm_read"):
            if key in e:
                e[key] = _median([r.get(key) for r in rows])
        e["parity_max_abs_err"] = max(r["parity_max_abs_err"] for r in rows)
        if len(rows) > 1:
            e["ms_median_per_process"] = [r["ms_median"] for r in rows]
        configs[name] = e
    traffic = traffic_from_counters(COUNTERS_FILE)
    dtraffic = traffic_from_counters(DECODE_COUNTERS_FILE)
    result = {
        "metric": "GQA prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM) on 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(_median([c["ms_per_step"] for c in children]), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V, decode lengths U[512,2048]",
        "config": {
            "workload": "llama3_8b_prefill + kv_decode_b8",
            "prefill": {"B": ps.B, "Hq": ps.Hq, "Hkv": ps.Hkv, "N": ps.Nq, "d": ps.d,
                        "causal": True, "algorithmic_gflop": round(flops / 1e9, 4)},
            "decode": {"B": ds.B, "Hq": ds.Hq, "Hkv": ds.Hkv, "Smax": ds.Smax, "d": ds.d,
                       "sum_seqlens": int(sum(lens)), "cache_sets": DECODE_SETS,
                       "algorithmic_mb": round(dbytes / 1e6, 4)},
        },
        "prefill": {"ms": round(pre_ms, 5), "tflops": round(tflops, 3),
                    "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "frac_measured_mfma_peak": round(tflops / peaks["mfma_bf16_tflops"], 4)},
        "decode": {"ms": round(dec_ms, 5), "value": round(gbps, 2), "unit": "GB/s",
                   "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                   "frac_measured_hbm_read": round(gbps / peaks["hbm_read_gbps"], 4),
                   "traffic": dtraffic,
                   "note": "part + merge launches, event-timed, HBM-cold caches"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "measured_peaks": peaks,
        "configs": configs,
        "protocol": {"processes": len(children),
                     "value_per_process": [round(flops / (c["prefill_ms"] * 1e-3) / 1e12, 3)
                                           for c in children],
                     "decode_gbps_per_process": [round(c["decode_gbps"], 2) for c in children],
                     "configs": "3 warm-ups, then 5 windows of >= 10 ms of back-to-back calls "
                                "behind a queued spin kernel; median and min per call",
                     "parity": "every config against the CPU fp64 oracle, every element, in "
                               "each process before its timing"},
        "wall_s_timed": round(_median([c["wall_s_timed"] for c in children]), 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    for c in children:
        if "cpu_baseline" in c:
            result["cpu_baseline"] = c["cpu_baseline"]
            break
    for c in children:
        if "other_workloads" in c:
            result["other_workloads"] = c["other_workloads"]
            break
    return result


# ---------------------------------------------------------------- counter summaries

def _counter_rows(directory: str):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    for path in files:
        with open(path) as f:
            yield from csv.DictReader(f)


def _kernel_kind(name: str):
    """The kernels the counter summaries cover, by launch: the LLaMA prefill
    (pair kernel), the d=64 sweep (persistent), the chunked prefill (quad),
    the batch-8 decode (part + merge), the calibration copy and the MFMA
    microbenchmark."""
    n = name.split("(")[0].replace("void ", "")
    if "neg_kernel" in name:
        return "copy"
    if "mfma_peak_kernel" in name:
        return "mfma_peak"
    for key in ("prefill_pair_kernel", "prefill_quad_kernel", "prefill_kernel",
                "decode_part_kernel", "decode_merge_kernel", "decode_stream_kernel"):
        if "gqa::" + key + "<" in n:
            return n
    return None


def _means(directory: str):
    """{(kernel, counter): mean per dispatch}, and mean duration per kernel (ns)."""
    vals, durs = {}, {}
    for row in _counter_rows(directory):
        kind = _kernel_kind(row["Kernel_Name"])
        if kind is None:
            continue
        vals.setdefault((kind, row["Counter_Name"]), []).append(float(row["Counter_Value"]))
        d = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        durs.setdefault(kind, []).append(d)
    return ({k: sum(v) / len(v) for k, v in vals.items()},
            {k: sum(v) / len(v) for k, v in durs.items()})


def summarize_counters(fetch_dir: str, write_dir: str, sq_dir: str):
    """HBM bytes per launch (FETCH_SIZE / WRITE_SIZE in KiB per dispatch, each
    scaled by what the counter reads for a plain copy of COPY_BYTES) for the
    LLaMA prefill and the batch-8 decode, and SQ counters per prefill kernel.
    Writes the JSON summaries bench.py reads and a markdown table."""
    from mqa_flashattention_amd.workloads import WORKLOADS, decode_inputs
    fetch, _ = _means(fetch_dir)
    write, _ = _means(write_dir)
    sq, durs = _means(sq_dir)
    read_factor = COPY_BYTES / (fetch[("copy", "FETCH_SIZE")] * 1024.0)
    write_factor = COPY_BYTES / (write[("copy", "WRITE_SIZE")] * 1024.0)

    def bytes_of(kinds):
        r = sum(fetch.get((k, "FETCH_SIZE"), 0.0) for k in kinds) * 1024.0 * read_factor
        w = sum(write.get((k, "WRITE_SIZE"), 0.0) for k in kinds) * 1024.0 * write_factor
        return r, w

    kinds = sorted({k for k, _ in fetch})
    pair = [k for k in kinds if "prefill_pair_kernel" in k and "128, 32, 4, false>, true" in k]
    dec = [k for k in kinds if ("decode_part_kernel" in k or "decode_merge_kernel" in k)
           and "128" in k and "true>" not in k]
    src_hash = kernel_source_hash()
    ps = WORKLOADS["llama3_8b_prefill"].fwd[0]
    ds = WORKLOADS["kv_decode_b8"].decode
    r, w = bytes_of(pair)
    prefill = {"kernel": " + ".join(pair), "workload": "llama3_8b_prefill (B1 Hq32 Hkv8 N2048 d128 "
               "causal, bf16)", "read_bytes_per_launch": round(r), "write_bytes_per_launch": round(w),
               "traffic_bytes_per_launch": round(r + w),
               "algorithmic_bytes_per_launch": round(fwd_bytes(ps)),
               "read_scale": round(read_factor, 4), "write_scale": round(write_factor, 4),
               "kernel_source_hash": src_hash}
    r, w = bytes_of(dec)
    lens = decode_inputs(ds, 0)[3].tolist()
    decode = {"kernel": " + ".join(dec), "workload": "kv_decode_b8 (B8 Hq12 Hkv2 Smax2048 d128, "
              "bf16, seed-0 lengths)", "read_bytes_per_launch": round(r),
              "write_bytes_per_launch": round(w), "traffic_bytes_per_launch": round(r + w),
              "algorithmic_bytes_per_launch": round(decode_bytes(ds, lens)),
              "read_scale": round(read_factor, 4), "write_scale": round(write_factor, 4),
              "per_kernel": {k: {"read_bytes": round(fetch.get((k, "FETCH_SIZE"), 0) * 1024 * read_factor),
                                 "write_bytes": round(write.get((k, "WRITE_SIZE"), 0) * 1024 * write_factor)}
                             for k in dec},
              "kernel_source_hash": src_hash}
    # SQ counters: MFMA-busy share = SQ_VALU_MFMA_BUSY_CYCLES over (SIMDs x the
    # per-XCD GRBM_GUI_ACTIVE, which rocprofv3 sums over the 8 XCDs)
    simds = 4 * 256
    sq_rows = {}
    for k in sorted({k for k, _ in sq}):
        g = sq.get((k, "GRBM_GUI_ACTIVE"))
        busy = sq.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"))
        mf = sq.get((k, "SQ_INSTS_MFMA"))
        va = sq.get((k, "SQ_INSTS_VALU"))
        lds = sq.get((k, "SQ_INSTS_LDS"))
        conf = sq.get((k, "SQ_LDS_BANK_CONFLICT"))
        sq_rows[k] = {
            "duration_us": round(durs.get(k, 0) / 1000, 2),
            "mfma_busy": round(busy / (simds * g / 8), 4) if busy and g else None,
            "valu_per_mfma": round(va / mf, 2) if va and mf else None,
            "lds_insts": round(lds) if lds is not None else None,
            "lds_bank_conflict_cycles": round(conf) if conf is not None else None,
            "conflict_cycles_per_lds_inst": round(conf / lds, 3) if conf is not None and lds else None,
            "waves": round(sq.get((k, "SQ_WAVES"), 0)),
            "gui_active_cycles_per_xcd": round(g / 8) if g else None}
    os.makedirs(PROFILES, exist_ok=True)
    _write_counter_markdown(prefill, decode, sq_rows, fetch_dir, write_dir, sq_dir)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(prefill, f, indent=1)
        f.write("\n")
    with open(DECODE_COUNTERS_FILE, "w") as f:
        json.dump(decode, f, indent=1)
        f.write("\n")
    with open(os.path.join(PROFILES, "sq_counters.json"), "w") as f:
        json.dump({"kernels": sq_rows, "kernel_source_hash": src_hash}, f, indent=1)
        f.write("\n")
    return {"prefill": prefill, "decode": decode, "sq": sq_rows}


COUNTER_CMD = ("cd /tmp && rocprofv3 --pmc {counters} --output-format csv -d <repo>/{out} -o p "
               "-- python3 <repo>/bench.py --counters-run --steps 3 --warmup 1")
SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
               "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def _short(kernel: str) -> str:
    """A readable kernel name: gqa::name<dtype, d, tile keys, waves, ...>."""
    import re
    m = re.match(r"gqa::(\w+)<(.*)>$", kernel)
    if not m:
        return kernel
    name, args = m.groups()
    args = args.replace("unsigned short", "bf16").replace("gqa::", "")
    return f"{name}<{args}>"


def _write_counter_markdown(prefill, decode, sq_rows, fetch_dir, write_dir, sq_dir):
    lines = ["# HBM traffic and SQ counters (rocprofv3 --pmc)", "",
             "Made by three counter runs of the same program, one pass each (a run can hold "
             "at most 4 TCC counters, and FETCH_SIZE uses 3 of them):", "",
             "    " + COUNTER_CMD.format(counters="FETCH_SIZE", out=fetch_dir),
             "    " + COUNTER_CMD.format(counters="WRITE_SIZE", out=write_dir),
             "    " + COUNTER_CMD.format(counters=SQ_COUNTERS, out=sq_dir),
             "    python3 bench.py --summarize-counters " + " ".join((fetch_dir, write_dir, sq_dir)),
             "",
             "`--counters-run` runs the step loop, then every configuration's kernels a few "
             "times, the 256 MiB calibration copy (torch.neg) and the MFMA microbenchmark.", "",
             "## HBM bytes per launch", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the counter "
             f"reads for the calibration copy of 256 MiB in and out: read x{prefill['read_scale']}, "
             f"write x{prefill['write_scale']} (FETCH_SIZE counts half the bytes read).", "",
             "| launch | kernels | read MB | write MB | total MB | algorithmic MB | ratio |",
             "|---|---|---|---|---|---|---|"]
    for label, r in (("LLaMA-3-8B causal prefill", prefill), ("batch-8 KV decode", decode)):
        lines.append(f"| {label} | {' + '.join(_short(k) for k in r['kernel'].split(' + '))} | "
                     f"{r['read_bytes_per_launch'] / 1e6:.3f} | {r['write_bytes_per_launch'] / 1e6:.3f} | "
                     f"{r['traffic_bytes_per_launch'] / 1e6:.3f} | "
                     f"{r['algorithmic_bytes_per_launch'] / 1e6:.3f} | "
                     f"{r['traffic_bytes_per_launch'] / r['algorithmic_bytes_per_launch']:.3f} |")
    lines += ["", "Decode per kernel:", "", "| kernel | read MB | write MB |", "|---|---|---|"]
    for k, v in decode["per_kernel"].items():
        lines.append(f"| {_short(k)} | {v['read_bytes'] / 1e6:.3f} | {v['write_bytes'] / 1e6:.3f} |")
    lines += ["", "## SQ counters per dispatch", "",
              "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE per XCD; "
              "rocprofv3 sums GRBM_GUI_ACTIVE over the 8 XCDs).  The MFMA microbenchmark row "
              "calibrates it (a register-only MFMA stream).", "",
              "| kernel | us | MFMA busy | VALU / MFMA | LDS insts | bank-conflict cycles | "
              "conflict cycles / LDS inst | waves |", "|---|---|---|---|---|---|---|---|"]
    for k, v in sq_rows.items():
        lines.append(f"| {_short(k)} | {v['duration_us']} | {v['mfma_busy']} | {v['valu_per_mfma']} | "
                     f"{v['lds_insts']} | {v['lds_bank_conflict_cycles']} | "
                     f"{v['conflict_cycles_per_lds_inst']} | {v['waves']} |")
    lines += ["", f"Kernel sources hash: {prefill['kernel_source_hash']}", ""]
    with open(os.path.join(PROFILES, "counters_hbm_and_sq.md"), "w") as f:
        f.write("\n".join(lines))


def summarize_trace(stats_csv: str, command: str, out_name: str):
    """A markdown table of one rocprofv3 --kernel-trace --stats run."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if "gqa::" not in r["Name"] and "_peak_kernel" not in r["Name"]:
                continue
            n = r["Name"].replace("(anonymous namespace)::", "")
            n = n.split("(")[0].replace("void ", "")
            rows.append((_short(n), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    lines = [f"# Kernel durations: {out_name}", "", "    " + command, "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for n, c, a, mi, ma in rows:
        lines.append(f"| {n} | {c} | {a:.2f} | {mi:.2f} | {ma:.2f} |")
    lines += ["", f"Kernel sources hash: {kernel_source_hash()}", ""]
    with open(os.path.join(PROFILES, out_name + ".md"), "w") as f:
        f.write("\n".join(lines))


# ---------------------------------------------------------------- entry

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--procs", type=int, default=3,
                    help="fresh child processes that each run the whole measurement (the "
                         "median is reported); 1 = run in this process (for profilers)")
    ap.add_argument("--all", action="store_true",
                    help="also time the token-major prefill, decode with append, the decode "
                         "graph replay, the backward, the mixed batches and the decode sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, stream 256 MiB through a plain elementwise kernel "
                         "twice (byte-counter calibration)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "SQ_DIR"),
                    help="write the counter summaries from three rocprofv3 --pmc outputs")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "COMMAND", "NAME"),
                    help="write profiles/NAME.md from a rocprofv3 kernel_stats.csv made by COMMAND")
    ap.add_argument("--counters-run", action="store_true",
                    help="in this process: parity, the step loop, then every config's kernels "
                         "a few times without timing windows (for rocprofv3 --pmc)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="time the LDS access patterns of the kernels' tile reads and staging "
                         "writes (libgqa_microbench.so) and print them as JSON lines")
    ap.add_argument("--valu-probe", action="store_true",
                    help="time fp32 FMA and exp2 chains (libgqa_microbench.so) and print the "
                         "lane operations per clock per CU as JSON lines")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-baseline", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args(argv)

    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters)))
        return 0
    if args.summarize_trace:
        stats, command, name = args.summarize_trace
        summarize_trace(stats, command, name)
        return 0

    if args.lds_probe:
        for row in lds_probe():
            print(json.dumps(row), flush=True)
        return 0
    if args.valu_probe:
        for row in valu_probe():
            print(json.dumps(row), flush=True)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention "
              "path is not sharded across GPUs by this library.", file=sys.stderr)
        return 2

    if args.child:
        res = run_child(args)
        print(CHILD_TAG + json.dumps(res), flush=True)
        return 0

    if args.counters_run:
        args.cpu_baseline = False
        args.calibration_copy = True
        run_child(args)
        print("# counters run done", flush=True)
        return 0
    if args.procs <= 1:
        args.cpu_baseline = not args.no_cpu_baseline
        children = [run_child(args)]
    else:
        # Fresh child processes, started here; this process never touches the GPU.
        children = []
        for i in range(args.procs):
            cmd = [sys.executable, os.path.abspath(__file__), "--child", "--steps", str(args.steps),
                   "--warmup", str(args.warmup)]
            if i == 0 and not args.no_cpu_baseline:
                cmd.append("--cpu-baseline")
            if i == 0 and args.all:
                cmd.append("--all")
            if args.calibration_copy:
                cmd.append("--calibration-copy")
            print(f"# bench process {i + 1}/{args.procs}", file=sys.stderr, flush=True)
            p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if p.returncode != 0:
                print(p.stdout[-2000:], file=sys.stderr)
                return p.returncode
            line = [ln for ln in p.stdout.splitlines() if ln.startswith(CHILD_TAG)]
            if not line:
                raise SystemExit("a bench process printed no result")
            children.append(json.loads(line[-1][len(CHILD_TAG):]))
    print(json.dumps(report(children, args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
