"""GPU parity of the packed variable-length forward (gqa_attn_fwd_varlen)
against the CPU oracle's per-sequence composition, element by element.

Bar as the other forward tests: max |O_gpu - O_oracle| <= 1e-4 for fp32
inputs and <= 2e-2 for bf16.  Cases: ragged mixes spanning several query
blocks and key tiles with ragged tails, empty and one-token sequences,
sequences with more queries than keys (causal rows that see no key come out
zero), sequences with no keys, MHA / GQA / MQA, every head dim, and the
mixed-length prompt batch at full size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_fwd_varlen
from mqa_flashattention_amd.workloads import VARLEN_PREFILL, varlen_inputs, varlen_lengths

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _run(lq, lk, Hq, Hkv, d, dtype, causal, seed=0, max_q=None, poison=False):
    q, k, v, cq, ck = varlen_inputs(lq, lk, Hq, Hkv, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    out = None
    if poison:  # every row must be written, the keyless ones with zeros
        out = torch.full(q.shape, float("nan"), dtype=dtype, device=DEV)
    got = attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV),
                          max_q if max_q is not None else max(max(lq), 1),
                          causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    ref = oracle.attn_fwd_varlen(q, k, v, cq.numpy(), ck.numpy(), causal=causal, scale=scale)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    print(f"varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}: "
          f"max abs error {err:.3g}")
    assert err <= TOL[dtype], err
    return got, ref, cq, ck


# (lens_q, lens_k): ragged tails, empty and one-token sequences, Nq > Nk,
# Nk = 0, and sequences spanning several 128-row query blocks and 64-key tiles
RAGGED = [
    ([5, 0, 7, 1, 3, 130], [9, 3, 3, 0, 3, 200]),
    ([257, 64, 1, 300], [257, 64, 1, 300]),          # whole prompts
    ([100, 200, 33], [40, 200, 1000]),                # chunks; the first has Nq > Nk
    ([1], [1]),
]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_varlen_ragged(case, causal, dtype, d):
    lq, lk = RAGGED[case]
    _run(lq, lk, 8, 2, d, dtype, causal, seed=case, poison=True)


@pytest.mark.parametrize("Hkv", [8, 2, 1], ids=["mha", "gqa", "mqa"])
def test_varlen_head_modes(Hkv):
    _run([77, 513, 2, 190], [77, 600, 2, 190], 8, Hkv, 64, torch.bfloat16, True, seed=3)


@pytest.mark.parametrize("Hq,Hkv", [(40, 1), (160, 1)], ids=["g40", "g160"])
def test_varlen_large_groups(Hq, Hkv):
    """Groups wider than a unit's 128 columns (several head blocks per K/V head)."""
    _run([33, 200, 5], [33, 260, 5], Hq, Hkv, 128, torch.bfloat16, True, seed=6)


def test_varlen_keyless_rows_are_zero():
    """Causal rows i < Nq - Nk see no key; a sequence with Nk = 0 has none."""
    got, _, cq, ck = _run([40, 6, 9], [10, 0, 9], 4, 2, 64, torch.bfloat16, True, seed=5,
                          poison=True)
    assert np.all(got[0:30] == 0.0)           # first sequence: rows 0..29 see no key
    assert np.any(got[30:40] != 0.0)
    assert np.all(got[40:46] == 0.0)          # second sequence: no keys at all


def test_varlen_max_seqlen_larger_than_needed():
    """A max_seqlen_q above every sequence's count only adds empty units."""
    _run([65, 3], [65, 3], 4, 1, 128, torch.bfloat16, True, seed=9, max_q=1000)


def test_varlen_matches_padded_forward_per_sequence():
    """Each sequence equals the dense forward of its own rows (chunk at
    q_offset Nk - Nq), computed by gqa_attn_fwd on the GPU."""
    from mqa_flashattention_amd import attn_fwd
    lq, lk = [130, 64, 200], [300, 64, 200]
    q, k, v, cq, ck = varlen_inputs(lq, lk, 8, 2, 128, torch.bfloat16, 11)
    out = attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), max(lq),
                          causal=True).cpu().double()
    for s in range(len(lq)):
        qs = q[cq[s]:cq[s + 1]].transpose(0, 1)[None].contiguous().to(DEV)
        ks = k[ck[s]:ck[s + 1]].transpose(0, 1)[None].contiguous().to(DEV)
        vs = v[ck[s]:ck[s + 1]].transpose(0, 1)[None].contiguous().to(DEV)
        dense = attn_fwd(qs, ks, vs, causal=True, q_offset=lk[s] - lq[s])
        dense = dense[0].transpose(0, 1).cpu().double()
        diff = float((dense - out[cq[s]:cq[s + 1]]).abs().max())
        assert diff <= 1e-2, (s, diff)


def test_varlen_prompt_batch_full():
    """Eight whole prompts of 128..2048 tokens (LLaMA-3-8B attention shape,
    causal, bf16), every element against the oracle."""
    s = VARLEN_PREFILL
    lens = varlen_lengths(s)
    _run(lens, lens, s.Hq, s.Hkv, s.d, s.dtype, s.causal, seed=0)


def test_varlen_repeatable():
    """Twenty reruns give the same bits (the schedule changes which
    workgroup runs a unit, not the unit's arithmetic)."""
    s = VARLEN_PREFILL
    lens = varlen_lengths(s, seed=1)[:4]
    q, k, v, cq, ck = [t.to(DEV) for t in varlen_inputs(lens, lens, s.Hq, s.Hkv, s.d, s.dtype, 1)]
    first = attn_fwd_varlen(q, k, v, cq, ck, max(lens), causal=True)
    for _ in range(20):
        again = attn_fwd_varlen(q, k, v, cq, ck, max(lens), causal=True)
        assert torch.equal(first, again)
