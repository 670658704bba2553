"""GPU parity of the strided forward (gqa_attn_fwd_strided).

The strided entry runs the same kernels on the same values as the
contiguous one, only addressing them through the caller's strides, so its
output must equal the contiguous call bit for bit.  That is checked on the
named workloads at full size in token-major (BTHD) layout -- one case per
prefill schedule (pair: LLaMA causal; persistent: MHA/GQA/MQA sweep;
balanced + merge: chunked prefill) -- and against the CPU fp64 oracle, to
the dtype tolerance, on small shapes with padded, permuted and broadcast
(zero) strides.  Padding between output rows must stay untouched.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_fwd, attn_fwd_strided
from mqa_flashattention_amd.workloads import WORKLOADS, FwdShape, fwd_inputs, random_tensor

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _bthd(x: torch.Tensor) -> torch.Tensor:
    """A token-major [B, N, H, d] copy of x [B, H, N, d], returned as the logical
    [B, H, N, d] view of it (strides {N*H*d, d, H*d})."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def _bitwise_case(s: FwdShape, seed: int):
    q, k, v = (t.to(DEV) for t in fwd_inputs(s, seed))
    ref = attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    qb, kb, vb = _bthd(q), _bthd(k), _bthd(v)
    out = attn_fwd_strided(qb, kb, vb, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    torch.cuda.synchronize()
    assert out.stride() == qb.stride()
    assert torch.equal(out, ref), f"{s}: strided output differs from the contiguous one"


def test_bthd_llama_prefill_bitwise():
    _bitwise_case(WORKLOADS["llama3_8b_prefill"].fwd[0], 0)


@pytest.mark.parametrize("variant", [0, 1, 2], ids=["mha_hkv16", "gqa_hkv4", "mqa_hkv1"])
def test_bthd_sweep_bitwise(variant):
    _bitwise_case(WORKLOADS["mha_gqa_mqa_sweep"].fwd[variant], 3)


def test_bthd_chunked_prefill_bitwise():
    _bitwise_case(WORKLOADS["chunked_prefill_4k"].fwd[0], 4)


@pytest.mark.parametrize("s", [FwdShape(1, 48, 12, 2000, 2000, 128, True, 0),
                               FwdShape(2, 32, 8, 256, 1000, 128, True, 744),
                               FwdShape(2, 32, 8, 2200, 2300, 128, False, 0),
                               FwdShape(4, 16, 4, 4000, 4000, 64, False, 0)],
                         ids=["pair", "quad", "persistent_d128", "persistent_d64"])
def test_bthd_ragged_keys_bitwise(s):
    """Key counts that end in a partial key tile, on the schedules that load K
    rows straight into LDS (pair, quad, non-causal persistent at d = 128 and
    64), through the token stride.  The shapes have enough units for the
    persistent schedule whatever the kernels' occupancy: the balanced
    schedule's chunk plan follows the resident workgroups, which may differ
    between the strided and contiguous kernels, and with it the summation
    order (both then stay within the oracle's bar, not bit for bit)."""
    _bitwise_case(s, 5)


def _padded(x: torch.Tensor, pad_h: int, pad_n: int, order=(0, 1, 2)):
    """x [B, H, N, d] copied into a bigger buffer whose (batch, head, token)
    dimensions are laid out in the given outer-to-inner order, with pad_h
    extra elements after each head block and pad_n after each token row.
    Returns (logical [B, H, N, d] view, whole buffer); the padding holds NaN."""
    B, H, N, d = x.shape
    ext = {0: B, 1: H, 2: N}
    pad = {0: 0, 1: pad_h, 2: pad_n}
    strides = {}
    inner = d
    for dim in reversed(order):
        strides[dim] = inner + pad[dim]
        inner = strides[dim] * ext[dim]
    buf = torch.full((inner,), float("nan"), dtype=x.dtype, device=x.device)
    view = buf.as_strided((B, H, N, d), (strides[0], strides[1], strides[2], 1))
    view.copy_(x)
    return view, buf


STRIDE_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal, q_offset, dtype, pad_h, pad_n, order)
    (2, 8, 2, 77, 77, 128, True, 0, torch.bfloat16, 64, 8, (0, 2, 1)),
    (1, 6, 6, 40, 130, 64, False, 0, torch.bfloat16, 0, 24, (0, 1, 2)),
    (2, 12, 2, 33, 97, 32, True, 64, torch.bfloat16, 16, 16, (2, 0, 1)),
    (1, 4, 1, 50, 50, 128, True, 0, torch.float32, 4, 4, (0, 2, 1)),
    (3, 40, 1, 20, 45, 64, True, 25, torch.bfloat16, 8, 0, (0, 2, 1)),
]


@pytest.mark.parametrize("case", STRIDE_CASES, ids=[f"case{i}" for i in range(len(STRIDE_CASES))])
def test_padded_strides_against_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, causal, off, dtype, pad_h, pad_n, order = case
    s = FwdShape(B, Hq, Hkv, Nq, Nk, d, causal, off, dtype)
    q, k, v = fwd_inputs(s, 11)
    qp, _ = _padded(q.to(DEV), pad_h, pad_n, order)
    kp, _ = _padded(k.to(DEV), pad_h, pad_n, order)
    vp, _ = _padded(v.to(DEV), pad_h, pad_n, order)
    out, obuf = _padded(torch.zeros_like(q, device=DEV), pad_h, pad_n, order)
    before = obuf.clone()
    attn_fwd_strided(qp, kp, vp, causal=causal, q_offset=off, scale=s.scale, out=out)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, scale=s.scale)
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[dtype], f"max abs error {err}"
    # every element of the buffer outside the output view still holds its NaN
    inside = torch.zeros(obuf.numel(), dtype=torch.bool, device=DEV)
    inside.as_strided(out.shape, out.stride()).fill_(True)
    assert bool(torch.all(torch.isnan(obuf[~inside]))), "output padding was written"
    assert torch.isnan(before[~inside]).all()


def test_broadcast_kv_over_batch():
    """A zero K/V batch stride reads one K/V for every batch row."""
    B, Hq, Hkv, N, d = 3, 8, 2, 70, 64
    q = random_tensor((B, Hq, N, d), 31, torch.bfloat16)
    k1 = random_tensor((1, Hkv, N, d), 32, torch.bfloat16)
    v1 = random_tensor((1, Hkv, N, d), 33, torch.bfloat16)
    kb = k1.to(DEV).expand(B, Hkv, N, d)
    vb = v1.to(DEV).expand(B, Hkv, N, d)
    assert kb.stride(0) == 0
    out = attn_fwd_strided(q.to(DEV), kb, vb, causal=True)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd(q, k1.expand(B, Hkv, N, d), v1.expand(B, Hkv, N, d), causal=True)
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    assert err <= TOL[torch.bfloat16], f"max abs error {err}"


def test_broadcast_kv_over_tokens():
    """A zero K/V token stride: every key row is the same row (expand over
    tokens), so each query's output is that V row exactly in exact arithmetic."""
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 50, 90, 128
    q = random_tensor((B, Hq, Nq, d), 41, torch.bfloat16)
    k1 = random_tensor((B, Hkv, 1, d), 42, torch.bfloat16)
    v1 = random_tensor((B, Hkv, 1, d), 43, torch.bfloat16)
    kb = k1.to(DEV).expand(B, Hkv, Nk, d)
    vb = v1.to(DEV).expand(B, Hkv, Nk, d)
    assert kb.stride(2) == 0
    for causal, off in ((False, 0), (True, 3)):
        out = attn_fwd_strided(q.to(DEV), kb, vb, causal=causal, q_offset=off)
        torch.cuda.synchronize()
        ref = oracle.attn_fwd(q, k1.expand(B, Hkv, Nk, d), v1.expand(B, Hkv, Nk, d),
                              causal=causal, q_offset=off)
        err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
        assert err <= TOL[torch.bfloat16], f"causal={causal}: max abs error {err}"


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_overlapping_kv_window(d, dtype):
    """K/V rows that overlap: key row j is elements [j*d/2, j*d/2 + d) of one
    flat buffer per head (a token stride of half a row)."""
    B, Hq, Hkv, Nq, Nk = 1, 4, 2, 40, 77
    esz = 2 if dtype == torch.bfloat16 else 4
    step = d // 2
    assert (step * esz) % 16 == 0
    flat_n = (Nk - 1) * step + d
    kf = random_tensor((B, Hkv, flat_n), 44, dtype).to(DEV)
    vf = random_tensor((B, Hkv, flat_n), 45, dtype).to(DEV)
    kw = kf.as_strided((B, Hkv, Nk, d), (Hkv * flat_n, flat_n, step, 1))
    vw = vf.as_strided((B, Hkv, Nk, d), (Hkv * flat_n, flat_n, step, 1))
    q = random_tensor((B, Hq, Nq, d), 46, dtype)
    out = attn_fwd_strided(q.to(DEV), kw, vw, causal=True, q_offset=Nk - Nq)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd(q, kw.cpu().contiguous(), vw.cpu().contiguous(), causal=True,
                          q_offset=Nk - Nq)
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    assert err <= TOL[dtype], f"max abs error {err}"
