"""The forwards under HIP-graph capture.

After one eager call with the same sizes on the capturing stream, a captured
gqa_attn_fwd (every schedule: persistent, causal pair, key-split quad,
balanced with partial records) or gqa_attn_fwd_varlen replays to the eager
bits: outputs are poisoned before each replay and eager calls run between
replays.  A call that would have to set up the stream's state while the
stream is capturing fails cleanly instead.
"""
from __future__ import annotations

import pytest
import torch

from mqa_flashattention_amd import attn_fwd, attn_fwd_varlen
from mqa_flashattention_amd.binding import GqaError
from mqa_flashattention_amd.workloads import WORKLOADS, FwdShape, fwd_inputs, varlen_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _replays_match_eager(call, outs, s):
    with torch.cuda.stream(s):
        call()
    s.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, ref))
        with torch.cuda.stream(s):
            call()
        s.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, ref))


FWD_CASES = {
    # persistent schedule: many units (the GQA variant of the head-mode sweep)
    "persistent": WORKLOADS["mha_gqa_mqa_sweep"].fwd[1],
    # causal pair schedule: the LLaMA-3-8B prefill shape
    "pair": WORKLOADS["llama3_8b_prefill"].fwd[0],
    # key-split quad schedule: a 512-query chunk at position 3584 of a 4096-token prompt
    "quad": WORKLOADS["chunked_prefill_4k"].fwd[0],
    # balanced schedule whose chunks cut units (partial records + merge)
    "balanced": FwdShape(1, 8, 2, 1024, 1024, 128, False, 0),
}


@pytest.mark.parametrize("name", list(FWD_CASES))
def test_fwd_graph_replay_matches_eager(name):
    sh = FWD_CASES[name]
    q, k, v = (t.to(DEV) for t in fwd_inputs(sh, 21))
    o = torch.empty_like(q)
    s = torch.cuda.Stream()
    _replays_match_eager(lambda: attn_fwd(q, k, v, causal=sh.causal, q_offset=sh.q_offset,
                                          scale=sh.scale, out=o), [o], s)


def test_varlen_graph_replay_matches_eager():
    lq = [300, 17, 1000, 64]
    q, k, v, cq, ck = (t.to(DEV) for t in varlen_inputs(lq, lq, 16, 4, 128, torch.bfloat16, 22))
    o = torch.empty_like(q)
    s = torch.cuda.Stream()
    _replays_match_eager(lambda: attn_fwd_varlen(q, k, v, cq, ck, max(lq), causal=True, out=o),
                         [o], s)


def test_graph_survives_a_later_larger_workspace():
    """A graph captured on the balanced schedule keeps replaying correctly after
    a larger eager call on the same stream has grown the stream's record
    buffer (the replaced buffer stays allocated)."""
    small = FwdShape(1, 8, 2, 512, 512, 128, False, 0)
    big = FwdShape(1, 8, 2, 1024, 1024, 128, False, 0)   # balanced, 4x the records
    q, k, v = (t.to(DEV) for t in fwd_inputs(small, 24))
    o = torch.empty_like(q)
    s = torch.cuda.Stream()

    def call():
        attn_fwd(q, k, v, scale=small.scale, out=o)

    with torch.cuda.stream(s):
        call()
    s.synchronize()
    ref = o.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    qb, kb, vb = (t.to(DEV) for t in fwd_inputs(big, 25))
    with torch.cuda.stream(s):
        ob = attn_fwd(qb, kb, vb, scale=big.scale)   # grows the record buffer
    s.synchronize()
    for _ in range(3):
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref)
    assert torch.isfinite(ob).all()


def test_capture_before_setup_fails_cleanly():
    """The first persistent call on a fresh stream must allocate its
    counters, which capture cannot hold: it fails and launches nothing; the
    same call outside capture then works."""
    sh = FWD_CASES["persistent"]
    q, k, v = (t.to(DEV) for t in fwd_inputs(sh, 23))
    o = torch.zeros_like(q)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(GqaError, match="captured"):
            attn_fwd(q, k, v, causal=sh.causal, scale=sh.scale, out=o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
    with torch.cuda.stream(s):
        attn_fwd(q, k, v, causal=sh.causal, scale=sh.scale, out=o)
    s.synchronize()
    assert torch.count_nonzero(o) > 0
