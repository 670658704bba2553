#!/usr/bin/env python3
"""Benchmark of the GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all]
    python bench.py --steps 5 --warmup 2 --no-cpu-baseline --calibration-copy
        (the run profiled with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR
        (turns those two rocprofv3 outputs into the committed counter summary)

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill: LLaMA-3-8B-shaped causal prefill, bf16 in / fp32 accumulate,
    B=1 Hq=32 Hkv=8 N=2048 d=128 (gqa_attn_fwd), and
  * decode:  KV-cache decode, bf16 cache, B=8 Hq=12 Hkv=2 d=128, lengths
    U[512, 2048] (gqa_attn_decode: split kernel + combine kernel).
Both are checked against the CPU oracle before anything is timed.

value = prefill TFLOP/s (algorithmic FLOPs = 4 * B * Hq * d * visible
(query, key) pairs, causal-masked pairs not counted) over the prefill
launch's event-timed average duration.  The decode part is reported beside
it in GB/s of algorithmic bytes (the K/V rows each sequence needs, plus q, o
and the lengths) over its event-timed duration; each decode call reads a
different one of several independently drawn caches so the reads come from
HBM, not from the 256 MB Infinity Cache.

`roofline` is for the prefill kernel (the dominant kernel of a step):
bf16 dense MFMA peak 2500 TFLOP/s.  `traffic` comes from the committed
rocprofv3 counter summary when it was taken from the current kernel sources,
else null.  `cpu_baseline` times the fp64 oracle on the host on the full
prefill workload.

Only one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefill_llama3_8b_counters.json")
KERNEL_SOURCES = ["attn_tile.hpp", "prefill_kernel.hpp", "decode_kernel.hpp", "mixed_kernel.hpp",
                  "backward_kernel.hpp", "gqa_attn.hip"]
DECODE_SETS = 48  # 48 x 16 MiB of caches > 256 MB Infinity Cache
COPY_BYTES = 256 * 1024 * 1024  # calibration copy: reads and writes this many bytes


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


def traffic_from_counters():
    """Measured HBM bytes per prefill launch, if the counters match the sources."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def _counter_means(directory: str, counter: str) -> dict:
    """Mean per-dispatch value of one rocprofv3 counter, by kernel kind: the
    d=128 bf16 causal prefill kernel(s) the bench workload launches, and the
    calibration copy.  Also returns the prefill kernel names seen."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    vals: dict = {}
    names: set = set()
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                # the LLaMA launch: bf16 d=128, 32-key tiles, contiguous K/V, causal
                if "gqa::prefill" in name and "128, 32, 4, false>, true" in name:
                    kind = name.split("(")[0].replace("void ", "")
                    names.add(kind)
                elif "neg_kernel" in name:
                    kind = "copy"
                else:
                    continue
                vals.setdefault(kind, []).append(float(row["Counter_Value"]))
    means = {k: sum(v) / len(v) for k, v in vals.items()}
    # one prefill launch = one dispatch of each prefill kernel it uses
    out = {"copy": means["copy"], "prefill": sum(means[n] for n in names),
           "names": sorted(names)}
    return out


def summarize_counters(fetch_dir: str, write_dir: str) -> dict:
    """HBM bytes per prefill launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    COPY_BYTES (read COPY_BYTES, write COPY_BYTES)."""
    from mqa_flashattention_amd.workloads import WORKLOADS
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    read_factor = COPY_BYTES / (fetch["copy"] * 1024.0)
    write_factor = COPY_BYTES / (write["copy"] * 1024.0)
    traffic = fetch["prefill"] * 1024.0 * read_factor + write["prefill"] * 1024.0 * write_factor
    out = {
        "kernel": ", ".join(fetch["names"]),
        "workload": "llama3_8b_prefill (B1 Hq32 Hkv8 N2048 d128 causal, bf16)",
        "fetch_kib_per_launch": round(fetch["prefill"], 1),
        "write_kib_per_launch": round(write["prefill"], 1),
        "copy_fetch_kib": round(fetch["copy"], 1),
        "copy_write_kib": round(write["copy"], 1),
        "read_scale": round(read_factor, 4),
        "write_scale": round(write_factor, 4),
        "traffic_bytes_per_launch": round(traffic),
        "algorithmic_bytes_per_launch": round(fwd_bytes(WORKLOADS["llama3_8b_prefill"].fwd[0])),
        "kernel_source_hash": kernel_source_hash(),
    }
    return out


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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true",
                    help="also time the MHA/GQA/MQA sweep, the chunked prefill, the "
                         "token-major prefill, decode with append, the backward and the "
                         "decode sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, stream 256 MiB through a plain elementwise kernel "
                         "twice (byte-counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the prefill counter summary from two rocprofv3 --pmc outputs")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        summary = summarize_counters(*args.summarize_counters)
        os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(summary, f, indent=1)
            f.write("\n")
        print(json.dumps(summary))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention "
              "path is not sharded across GPUs by this library.", file=sys.stderr)
        return 2

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

    flops = prefill_flops(ps)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    lens = dl_h.tolist()
    dbytes = decode_bytes(ds, lens)
    gbps = dbytes / (dec_ms * 1e-3) / 1e9

    result = {
        "metric": "GQA prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM) on 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
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
                    "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4)},
        "decode": {"ms": round(dec_ms, 5), "value": round(gbps, 2), "unit": "GB/s",
                   "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                   "note": "split + combine launches, event-timed, HBM-cold caches"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_counters()},
        "wall_s_timed": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = {
            "value": round(flops / oracle_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole prefill workload (B1 Hq32 Hkv8 N2048 d128 causal), fp64, "
                      f"{oracle_s:.2f} s wall",
            "decode_gbps": round(dbytes / oracle_dec_s / 1e9, 4),
        }

    if args.calibration_copy:
        # a plain streaming kernel of known traffic: reads and writes COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.all:
        extra = {}
        for name in ("mha_gqa_mqa_sweep", "chunked_prefill_4k"):
            for s in WORKLOADS[name].fwd:
                ms = time_fwd_workload(s, max(10, K // 2), 3)
                tf = prefill_flops(s) / (ms * 1e-3) / 1e12
                extra[f"{name}[Hkv={s.Hkv}]"] = {"ms": round(ms, 5), "tflops": round(tf, 2),
                                                 "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        ms = time_fwd_workload(ps, max(10, K // 2), 3, bthd=True)
        tf = prefill_flops(ps) / (ms * 1e-3) / 1e12
        extra["llama3_8b_prefill[bthd]"] = {
            "ms": round(ms, 5), "tflops": round(tf, 2),
            "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "note": "token-major [B, N, H, d] Q/K/V/O through gqa_attn_fwd_strided, no copies"}
        sa = WORKLOADS["kv_decode_append_b8"].decode
        ms, positions = time_append_workload(sa, max(20, K), 5)
        gb = append_bytes(sa, positions) / (ms * 1e-3) / 1e9
        extra["kv_decode_append_b8"] = {
            "ms": round(ms, 5), "value": round(gb, 2), "unit": "GB/s",
            "frac_hbm_peak": round(gb / PEAK_HBM_GBPS, 4),
            "algorithmic_mb": round(append_bytes(sa, positions) / 1e6, 4),
            "note": "store of the new K/V rows + split + combine, one call, HBM-cold caches"}
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
                    "dK/dV kernel (query range of each key block in up to 8 parts) and their "
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
                        "rows in one persistent launch + the decode combine, against gqa_attn_fwd "
                        "then gqa_attn_decode; decode caches HBM-cold"}
        extra.update(time_decode_sweep(20, 3))
        result["other_workloads"] = extra

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
