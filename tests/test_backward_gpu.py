"""GPU parity of the backward (gqa_attn_bwd) against the CPU fp64 oracle.

dQ, dK, dV from the HIP kernels (through the C ABI) are compared element by
element with oracle_attn_bwd on the same inputs: q, k, v and dout as the
kernels read them (bf16 or fp32, widened exactly), o from the library's own
forward.  Cases span MHA / GQA / MQA, every head dim, causal offsets, ragged
lengths, fp32 and bf16, and the LLaMA-3-8B prefill shape at full size.

Bar, for every element of all three gradients:
    |got - ref| <= atol + rtol * |ref|
atol is the forward's bound (1e-4 fp32, 2e-2 bf16).  Unlike the forward's
outputs, which never exceed max |V|, gradients are sums over every row of
a K/V head's group and reach magnitudes of several units; there the bf16
path's two roundings -- the MFMA operand P or dS, and the output itself,
each at most 2^-8 relative -- exceed any fixed absolute bound, so rtol is
2^-7 for bf16 and 1e-5 for fp32 (fp32 accumulation over up to 10^4 terms).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_bwd, attn_fwd
from mqa_flashattention_amd.workloads import WORKLOADS, FwdShape, fwd_inputs, random_tensor

pytestmark = pytest.mark.gpu

ATOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
RTOL = {torch.float32: 1e-5, torch.bfloat16: 2.0 ** -7}
DEV = "cuda:0"


def _run(s: FwdShape, seed: int):
    q, k, v = fwd_inputs(s, seed)
    do = random_tensor(q.shape, seed + 11, s.dtype)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o = attn_fwd(qd, kd, vd, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    grads = attn_bwd(qd, kd, vd, o, dod, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    torch.cuda.synchronize()
    return (q, k, v, do), (qd, kd, vd, o, dod), grads


def _check(s: FwdShape, seed: int = 0):
    (q, k, v, do), _, grads = _run(s, seed)
    want = oracle.attn_bwd(q, k, v, do, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        got = g.cpu().double().numpy()
        assert np.all(np.isfinite(got)), f"{name}: non-finite values"
        err = np.abs(got - w)
        excess = err - (ATOL[s.dtype] + RTOL[s.dtype] * np.abs(w))
        worst = np.unravel_index(int(np.argmax(excess)), excess.shape)
        print(f"{s} {name}: max abs error {float(err.max()):.3e} (max |ref| "
              f"{float(np.abs(w).max()):.3e}), max excess over atol + rtol|ref| "
              f"{float(excess[worst]):.3e}", flush=True)
        assert excess[worst] <= 0, (f"{s} {name}: error {abs(got[worst] - w[worst]):.3e} at "
                                    f"{worst} where |ref| = {abs(w[worst]):.3e}")


@pytest.mark.parametrize("s", [
    FwdShape(1, 4, 2, 64, 64, 32, False, 0, torch.float32),     # the tiny fp32 shape
    FwdShape(1, 4, 1, 33, 33, 32, True, 0, torch.float32),      # MQA, ragged
    FwdShape(2, 8, 2, 96, 70, 64, False, 0, torch.float32),     # Nq != Nk
    FwdShape(1, 4, 2, 45, 80, 128, True, 35, torch.float32),    # chunk at an offset
    FwdShape(2, 4, 4, 100, 100, 64, True, 0, torch.bfloat16),   # MHA, ragged
    FwdShape(1, 8, 2, 127, 127, 128, True, 0, torch.bfloat16),  # GQA, one short of a tile
    FwdShape(1, 6, 1, 40, 200, 128, True, 160, torch.bfloat16), # MQA, chunk at an offset
    FwdShape(1, 12, 2, 50, 300, 128, True, 250, torch.bfloat16),  # group of 6
    FwdShape(1, 8, 8, 70, 130, 32, False, 0, torch.bfloat16),
    FwdShape(1, 160, 1, 20, 90, 64, True, 70, torch.bfloat16),  # more heads than a unit
], ids=lambda s: f"B{s.B}_Hq{s.Hq}_Hkv{s.Hkv}_{s.Nq}x{s.Nk}_d{s.d}_"
                 f"{'c' + str(s.q_offset) if s.causal else 'full'}_{str(s.dtype)[6:]}")
def test_bwd_small_shapes(s):
    _check(s, seed=3)


def test_bwd_llama3_8b_shape_full():
    """The LLaMA-3-8B prefill shape (B1 Hq32 Hkv8 N2048 d128, causal, bf16),
    every element of dQ, dK and dV."""
    _check(WORKLOADS["llama3_8b_prefill"].fwd[0], seed=0)


# query parts per key block: min(16, ceil(1024 / key blocks)), with
# ceil(Nk / 64) key blocks per (batch, K/V head)
@pytest.mark.parametrize("s", [
    FwdShape(1, 16, 4, 2048, 2048, 64, True, 0),   # 128 key blocks: eight query parts
    FwdShape(1, 16, 8, 2048, 2048, 64, True, 0),   # 256: four
    FwdShape(1, 16, 16, 2048, 2048, 64, True, 0),  # 512: two
    FwdShape(4, 16, 16, 2048, 2048, 64, True, 0),  # 2048: one, dK and dV written directly
    FwdShape(1, 16, 8, 2048, 2048, 128, True, 0),  # d = 128 (the 16-key dK/dV kernel), four
    FwdShape(4, 16, 16, 2048, 2048, 128, True, 0),  # d = 128, one
], ids=["eight_parts", "four_parts", "two_parts", "one_part", "d128_four_parts",
        "d128_one_part"])
def test_bwd_query_split_counts(s):
    """Launches large enough that each key block's query range is cut into
    eight, four or two parts, or not cut at all (the small shapes above use
    sixteen); bf16 at d = 128 runs the 16-key dK/dV kernel, the others the
    32-key one."""
    _check(s, seed=5)


def test_bwd_offset_past_end_is_noncausal():
    """q_offset >= Nk - 1 sees every key: the causal call equals the full one."""
    s = FwdShape(1, 4, 2, 40, 64, 64, True, 80)
    _, (qd, kd, vd, o, dod), g1 = _run(s, 7)
    g2 = attn_bwd(qd, kd, vd, o, dod, causal=False, scale=s.scale)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_bitwise_deterministic():
    s = FwdShape(1, 8, 2, 300, 300, 128, True, 0)
    _, (qd, kd, vd, o, dod), g1 = _run(s, 9)
    for _ in range(5):
        g2 = attn_bwd(qd, kd, vd, o, dod, causal=True, scale=s.scale)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
    torch.cuda.synchronize()
