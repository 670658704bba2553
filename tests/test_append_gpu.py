"""GPU parity of the decode step with append (gqa_attn_decode_append).

Against the CPU fp64 oracle: outputs within the dtype tolerance (1e-4 fp32,
2e-2 bf16) and the updated caches bit-exact (the store is a copy).  The slot
each row writes is filled with NaN beforehand, and so are all slots past it,
so a kernel that read the stale slot or any slot beyond the row's position
would produce NaN.  Covers the batch-8 decode workload at full size,
positions on and around 32-token tile and split boundaries, the first and
last slot, inactive rows, more query heads per K/V head than one wave holds,
a multi-step decode loop, and bitwise agreement with storing first and then
calling the plain decode.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_decode, attn_decode_append, decode_workspace_bytes
from mqa_flashattention_amd.workloads import (WORKLOADS, DecodeShape, append_inputs,
                                              random_tensor)

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _poison(kc, vc, pos):
    """Copies of the caches with NaN in each active row's slot p and in every slot past it."""
    kp, vp = kc.clone(), vc.clone()
    Smax = kc.shape[2]
    for b, p in enumerate(pos.tolist()):
        if 0 <= p < Smax:
            kp[b, :, p:] = float("nan")
            vp[b, :, p:] = float("nan")
    return kp, vp


def _run(q, kn, vn, kc, vc, pos, scale=None):
    """One append step on the GPU; returns (out, kcache, vcache) on the CPU."""
    kd, vd = kc.to(DEV), vc.to(DEV)
    out = attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kd, vd, pos.to(DEV), scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), kd.cpu(), vd.cpu()


def _check(q, kn, vn, kc, vc, pos, scale=None):
    kp, vp = _poison(kc, vc, pos)
    out, ko, vo = _run(q, kn, vn, kp, vp, pos, scale)
    ref, kref, vref = oracle.attn_decode_append(q, kn, vn, kp, vp, pos, scale=scale)
    g = out.double().numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    err = float(np.max(np.abs(g - ref)))
    assert err <= TOL[q.dtype], f"max abs error {err}"
    assert np.array_equal(ko.double().numpy(), kref, equal_nan=True), "K cache differs"
    assert np.array_equal(vo.double().numpy(), vref, equal_nan=True), "V cache differs"
    return out


def _inputs(B, Hq, Hkv, Smax, d, dtype, seed):
    return (random_tensor((B, Hq, d), seed, dtype), random_tensor((B, Hkv, d), seed + 1, dtype),
            random_tensor((B, Hkv, d), seed + 2, dtype),
            random_tensor((B, Hkv, Smax, d), seed + 3, dtype),
            random_tensor((B, Hkv, Smax, d), seed + 4, dtype))


def test_append_workload_full():
    s = WORKLOADS["kv_decode_append_b8"].decode
    q, kn, vn, kc, vc, pos = append_inputs(s, 0)
    _check(q, kn, vn, kc, vc, pos, scale=s.scale)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_append_positions(dtype, d):
    """Positions on tile (32) and split boundaries, the first and last slot,
    and inactive rows (negative or at/after the capacity)."""
    Smax = 300
    pos = torch.tensor([0, 31, 32, 33, 63, 64, Smax - 1, -1, Smax, 150, -7, 1000, 95],
                       dtype=torch.int32)
    q, kn, vn, kc, vc = _inputs(len(pos), 6, 2, Smax, d, dtype, 40 + d)
    out = _check(q, kn, vn, kc, vc, pos)
    inactive = [i for i, p in enumerate(pos.tolist()) if not 0 <= p < Smax]
    assert torch.all(out[inactive] == 0)


@pytest.mark.parametrize("g", [40, 160])
def test_append_large_groups(g):
    """Several 32-head column blocks per K/V head: each patches its own tile,
    only the first stores."""
    pos = torch.tensor([0, 57, 89], dtype=torch.int32)
    q, kn, vn, kc, vc = _inputs(3, g, 1, 90, 64, torch.bfloat16, 70 + g)
    _check(q, kn, vn, kc, vc, pos)


def test_append_single_slot_cache():
    """Capacity 1: the only slot is the new token's, so the output is v_new."""
    pos = torch.tensor([0, 0, -1], dtype=torch.int32)
    q, kn, vn, kc, vc = _inputs(3, 4, 2, 1, 128, torch.bfloat16, 81)
    out = _check(q, kn, vn, kc, vc, pos)
    for h in range(4):
        assert torch.equal(out[:2, h], vn[:2, h // 2])


def test_append_decode_loop():
    """Four consecutive steps, each active row advancing one slot, one row
    inactive throughout; outputs and caches follow the oracle step by step."""
    B, Hq, Hkv, Smax, d = 5, 8, 2, 160, 128
    dtype = torch.bfloat16
    _, _, _, kc, vc = _inputs(B, Hq, Hkv, Smax, d, dtype, 90)
    pos = torch.tensor([0, 30, 63, 157, -1], dtype=torch.int32)
    kd, vd = kc.to(DEV), vc.to(DEV)
    kref, vref = kc.double().numpy(), vc.double().numpy()
    ws = torch.empty(decode_workspace_bytes(B, Hq, Hkv, Smax, d), dtype=torch.uint8, device=DEV)
    for step in range(4):
        q, kn, vn, _, _ = _inputs(B, Hq, Hkv, 1, d, dtype, 100 + 10 * step)
        out = attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kd, vd, pos.to(DEV),
                                 workspace=ws)
        torch.cuda.synchronize()
        ref, kref, vref = oracle.attn_decode_append(q, kn, vn, kref, vref, pos)
        err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
        assert err <= TOL[dtype], f"step {step}: max abs error {err}"
        pos = torch.where(pos >= 0, pos + 1, pos)
    assert np.array_equal(kd.cpu().double().numpy(), kref)
    assert np.array_equal(vd.cpu().double().numpy(), vref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_append_equals_store_then_decode(dtype):
    """The fused step gives bit-for-bit the output of writing the new rows
    into the caches first and then running the plain decode with
    seqlens = positions + 1 (same splits, same arithmetic)."""
    B, Hq, Hkv, Smax, d = 6, 12, 2, 700, 128
    pos = torch.tensor([0, 31, 255, 256, 699, 411], dtype=torch.int32)
    q, kn, vn, kc, vc = _inputs(B, Hq, Hkv, Smax, d, dtype, 120)
    out, _, _ = _run(q, kn, vn, kc, vc, pos)
    ks, vs = kc.clone(), vc.clone()
    for b, p in enumerate(pos.tolist()):
        ks[b, :, p] = kn[b]
        vs[b, :, p] = vn[b]
    ref = attn_decode(q.to(DEV), ks.to(DEV), vs.to(DEV), (pos + 1).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, ref.cpu())


@pytest.mark.parametrize("B,Hq,Hkv,Smax,d", [(40, 12, 2, 1500, 128), (20, 40, 1, 2000, 64)],
                         ids=["gqa6_d128", "g40_d64"])
def test_append_large_batches(B, Hq, Hkv, Smax, d):
    """Larger batches (several parts per row, several rounds of workgroups):
    positions on part and tile boundaries, inactive rows first, in the middle
    and last."""
    g = torch.Generator().manual_seed(B + Smax)
    pos = torch.randint(0, Smax, (B,), generator=g, dtype=torch.int32)
    special = [-1, 0, 31, 32, 127, 128, 255, 256, Smax - 1, Smax, -5, 1000 * Smax]
    pos[:len(special)] = torch.tensor(special, dtype=torch.int32)
    pos[B // 2] = -1
    pos[B - 1] = Smax + 3
    q, kn, vn, kc, vc = _inputs(B, Hq, Hkv, Smax, d, torch.bfloat16, 150 + d)
    out = _check(q, kn, vn, kc, vc, pos)
    inactive = [i for i, p in enumerate(pos.tolist()) if not 0 <= p < Smax]
    assert torch.all(out[inactive] == 0)
