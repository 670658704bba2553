"""GPU parity of the mixed batch (gqa_attn_mixed) against the CPU fp64 oracle.

One launch runs a chunked-prefill chunk (causal, query row i at position
q_offset + i) and decode rows of the same layer; both outputs are compared
element by element with oracle.attn_mixed on the same inputs.  Bar: the
forward's, max |O_gpu - O_oracle| <= 1e-4 for fp32 and <= 2e-2 for bf16.
Cases span every head dim, MHA / GQA / MQA and groups wider than one column
block, the three chunk schedules (the balanced schedule's key-tile chunks
with cut units merged after the launch, for chunks of few units -- every
small case; quad units for chunks of few long units, as a prefill call of
that shape takes them; 128-column persistent units for chunks of many
units), ragged chunk and cache lengths (empty, one slot, full capacity), a
missing part, both LLaMA-3-8B mixed workloads at full size, the decode
rows' agreement with gqa_attn_decode (bitwise where they use its splits)
and the quad chunk's bitwise identity with gqa_attn_fwd, determinism, and
back-to-back calls of different sizes sharing one stream's scheduler
counters.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_decode, attn_fwd, attn_mixed, decode_workspace_bytes
from mqa_flashattention_amd.workloads import (WORKLOADS, DecodeShape, FwdShape, fwd_inputs,
                                              mixed_inputs)

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().to("cpu").double().numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def _dev(ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _run(c: FwdShape, r: DecodeShape, seed: int, lens=None):
    q, k, v, qd, kc, vc, sl = mixed_inputs(c, r, seed)
    if lens is not None:
        sl = torch.tensor(lens, dtype=torch.int32)
    o, od = attn_mixed(*_dev((q, k, v)), c.q_offset, *_dev((qd, kc, vc, sl)), scale=c.scale)
    torch.cuda.synchronize()
    ro, rod = oracle.attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
    eo, eod = _err(o, ro), _err(od, rod)
    assert eo <= TOL[c.dtype], f"chunk {c}: max abs error {eo}"
    assert eod <= TOL[c.dtype], f"decode {r}: max abs error {eod}"
    return (q, k, v, qd, kc, vc, sl), o, od


def _pair(B, Hq, Hkv, Nq, Nk, off, Bd, Smax, lo, hi, d, dtype):
    return (FwdShape(B, Hq, Hkv, Nq, Nk, d, True, off, dtype),
            DecodeShape(Bd, Hq, Hkv, Smax, d, lo, hi, dtype))


SMALL = [
    _pair(1, 4, 2, 45, 80, 35, 3, 100, 1, 100, 32, torch.float32),
    _pair(2, 8, 2, 100, 300, 200, 5, 700, 1, 700, 64, torch.bfloat16),
    _pair(1, 12, 2, 70, 150, 80, 4, 2048, 1, 2048, 128, torch.bfloat16),     # group of 6
    _pair(1, 8, 1, 33, 33, 0, 6, 257, 200, 257, 128, torch.bfloat16),       # MQA, prompt start
    _pair(2, 4, 4, 64, 96, 32, 2, 96, 90, 96, 128, torch.float32),          # MHA
    _pair(1, 40, 1, 20, 90, 70, 3, 300, 1, 300, 32, torch.bfloat16),        # g = 40: 2 blocks
    # chunks of few long units: balanced pieces, every unit cut
    _pair(3, 16, 4, 127, 1000, 873, 9, 1000, 1, 1000, 64, torch.float32),
    _pair(1, 16, 2, 128, 1024, 896, 4, 1024, 1, 1024, 64, torch.bfloat16),  # group of 8
    _pair(2, 4, 1, 64, 800, 736, 3, 800, 1, 800, 32, torch.bfloat16),
    # 192 64-column units of >= 8 key tiles: quad units, as a prefill call takes them
    _pair(1, 16, 4, 768, 1536, 768, 5, 1536, 1, 1536, 64, torch.bfloat16),
]


@pytest.mark.parametrize("c,r", SMALL, ids=lambda x: (
    f"B{x.B}_Hq{x.Hq}_Hkv{x.Hkv}_{x.Nq}x{x.Nk}_c{x.q_offset}_d{x.d}_{str(x.dtype)[6:]}"
    if isinstance(x, FwdShape) else f"Bd{x.B}_S{x.Smax}"))
def test_mixed_small(c, r):
    _run(c, r, seed=2)


def test_mixed_empty_one_slot_and_full_rows():
    """Decode rows of length 0 (zero output), 1, Smax, and past Smax (clamped)."""
    c, r = _pair(1, 8, 2, 50, 120, 70, 5, 160, 1, 160, 128, torch.bfloat16)
    _, _, od = _run(c, r, seed=4, lens=[0, 1, 160, 999, -3])
    assert torch.all(od[0] == 0) and torch.all(od[4] == 0)


def test_mixed_one_part_missing():
    c, r = _pair(1, 8, 2, 96, 160, 64, 4, 512, 1, 512, 64, torch.bfloat16)
    q, k, v, qd, kc, vc, sl = mixed_inputs(c, r, 6)
    o, none_d = attn_mixed(*_dev((q, k, v)), c.q_offset, None, None, None, None, scale=c.scale)
    none_c, od = attn_mixed(None, None, None, 0, *_dev((qd, kc, vc, sl)), scale=c.scale)
    torch.cuda.synchronize()
    assert none_d is None and none_c is None
    ro, rod = oracle.attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
    assert _err(o, ro) <= TOL[c.dtype] and _err(od, rod) <= TOL[c.dtype]


@pytest.mark.parametrize("chunk", [False, True], ids=["decode_only", "short_chunk"])
def test_mixed_decode_rows_equal_decode_bitwise(chunk):
    """Without a chunk, or with one whose units leave workgroups free, the
    decode rows use gqa_attn_decode's splits, split code and combine pass:
    identical bits."""
    w = WORKLOADS["llama3_8b_mixed_c128"]
    c = w.fwd[0]
    q, k, v, qd, kc, vc, sl = _dev(mixed_inputs(c, w.decode, 12))
    if not chunk:
        q = k = v = None
    o, od = attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
    ref = attn_decode(qd, kc, vc, sl, scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(od, ref)
    assert (o is None) == (not chunk)


def test_llama3_8b_mixed_full():
    """The LLaMA-3-8B mixed workload at full size, every output element."""
    w = WORKLOADS["llama3_8b_mixed"]
    _run(w.fwd[0], w.decode, seed=0)


def test_llama3_8b_mixed_c128_full():
    """The 128-query mixed workload at full size (balanced pieces on half the
    workgroups, every unit cut), every output element."""
    w = WORKLOADS["llama3_8b_mixed_c128"]
    _run(w.fwd[0], w.decode, seed=1)


def test_mixed_many_units_persistent():
    """A chunk of 640 128-column units (more than the balanced schedule takes):
    the persistent units, then the decode parts."""
    c, r = _pair(1, 32, 8, 2560, 3072, 512, 4, 1024, 1, 1024, 128, torch.bfloat16)
    _run(c, r, seed=5)


def test_mixed_decode_rows_match_decode():
    """The decode rows run the decode kernel's split code (on shorter splits)
    and its combine pass: they agree with gqa_attn_decode to within the bar,
    and exactly where a row fits one split of either."""
    w = WORKLOADS["llama3_8b_mixed"]
    q, k, v, qd, kc, vc, sl = _dev(mixed_inputs(w.fwd[0], w.decode, 3))
    _, od = attn_mixed(q, k, v, w.fwd[0].q_offset, qd, kc, vc, sl, scale=w.fwd[0].scale)
    ref = attn_decode(qd, kc, vc, sl, scale=w.fwd[0].scale)
    torch.cuda.synchronize()
    assert float((od.double() - ref.double()).abs().max()) <= TOL[w.decode.dtype]
    one = torch.tensor([1, 5, 31, 32, 7, 2, 9, 17], dtype=torch.int32, device=DEV)
    _, od1 = attn_mixed(q, k, v, w.fwd[0].q_offset, qd, kc, vc, one, scale=w.fwd[0].scale)
    ref1 = attn_decode(qd, kc, vc, one, scale=w.fwd[0].scale)
    torch.cuda.synchronize()
    assert torch.equal(od1, ref1)


def test_mixed_chunk_equals_forward_bitwise():
    """The LLaMA-3-8B chunk has few long units, so both gqa_attn_mixed and
    gqa_attn_fwd run it as the same quad units over the same key ranges:
    identical bits."""
    w = WORKLOADS["llama3_8b_mixed"]
    c = w.fwd[0]
    q, k, v, qd, kc, vc, sl = _dev(mixed_inputs(c, w.decode, 7))
    o, _ = attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
    ref = attn_fwd(q, k, v, causal=True, q_offset=c.q_offset, scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_mixed_bitwise_deterministic():
    c, r = _pair(2, 32, 8, 300, 2000, 1700, 8, 2048, 1, 2048, 128, torch.bfloat16)
    q, k, v, qd, kc, vc, sl = _dev(mixed_inputs(c, r, 8))
    o1, od1 = attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
    for _ in range(10):
        o2, od2 = attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
        assert torch.equal(o1, o2) and torch.equal(od1, od2)
    torch.cuda.synchronize()


def test_mixed_calls_of_different_sizes_share_counters():
    """Mixed, forward and mixed calls back to back on one stream, large then
    small then large: each launch leaves the scheduler counters at zero for
    the next, so every call covers all its units and splits."""
    big = _pair(1, 32, 8, 512, 4096, 3584, 8, 4096, 512, 4096, 128, torch.bfloat16)
    small = _pair(1, 8, 2, 40, 64, 24, 2, 64, 1, 64, 64, torch.bfloat16)
    fwd_s = FwdShape(2, 32, 8, 2048, 2048, 128, True, 0)
    outs = []
    for i, (c, r) in enumerate((big, small, big)):
        ins = mixed_inputs(c, r, 20 + i)
        o, od = attn_mixed(*_dev(ins[:3]), c.q_offset, *_dev(ins[3:]), scale=c.scale)
        fq, fk, fv = fwd_inputs(fwd_s, 30 + i)
        fo = attn_fwd(*_dev((fq, fk, fv)), causal=True, scale=fwd_s.scale)
        outs.append((c, r, ins, o, od, (fq, fk, fv), fo))
    torch.cuda.synchronize()
    for c, r, ins, o, od, (fq, fk, fv), fo in outs:
        q, k, v, qd, kc, vc, sl = ins
        ro, rod = oracle.attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale)
        assert _err(o, ro) <= TOL[c.dtype] and _err(od, rod) <= TOL[c.dtype]
        ids = np.array([0, 2047, 32 * 2048 + 5, 2 * 32 * 2048 - 1])
        rf = oracle.attn_fwd_rows(fq, fk, fv, ids, causal=True, scale=fwd_s.scale)
        assert _err(fo.reshape(-1, 128)[torch.from_numpy(ids).to(DEV)], rf) <= TOL[fwd_s.dtype]


def test_mixed_graph_replay_matches_eager():
    """A serving loop may capture the mixed call in a HIP graph.  One eager
    call on the capture stream first sets up that stream's scheduler
    counters (the only allocation); the captured launches then replay, each
    leaving the counters at zero for the next.  Every replay, with outputs
    poisoned before it and eager calls between replays, gives the eager bits."""
    w = WORKLOADS["llama3_8b_mixed_c128"]
    c, r = w.fwd[0], w.decode
    q, k, v, qd, kc, vc, sl = _dev(mixed_inputs(c, r, 14))
    ws = torch.empty(decode_workspace_bytes(r.B, r.Hq, r.Hkv, r.Smax, r.d), dtype=torch.uint8,
                     device=DEV)
    o, od = torch.empty_like(q), torch.empty_like(qd)
    s = torch.cuda.Stream()

    def call():
        attn_mixed(q, k, v, c.q_offset, qd, kc, vc, sl, scale=c.scale, out=o, out_decode=od,
                   workspace=ws)

    with torch.cuda.stream(s):
        call()
    s.synchronize()
    ref_o, ref_od = o.clone(), od.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(4):
        o.fill_(float("nan"))
        od.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(od, ref_od)
        with torch.cuda.stream(s):
            call()
        s.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(od, ref_od)
