"""GPU parity of decode through a slot table (gqa_attn_decode_slots) against
the CPU oracle, element by element.

Bar: max |O_gpu - O_oracle| <= 2e-2 for bf16 and 1e-4 for fp32; inactive
rows (slot outside the pool) exactly zero; appended pools equal to the
oracle's bit for bit (the new rows are copies).  Cases: permuted, shared and
out-of-pool slots, lengths 0 .. Smax, append into distinct slots, the
identity table against gqa_attn_decode / _append bit for bit, relabelling
the pool (bit for bit), and a large pool at full decode sizes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_decode, attn_decode_append, attn_decode_slots
from mqa_flashattention_amd.workloads import random_tensor

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _pool(ncache, Hkv, Smax, d, dtype, seed):
    return (random_tensor((ncache, Hkv, Smax, d), seed, dtype),
            random_tensor((ncache, Hkv, Smax, d), seed + 1, dtype))


def _slots(B, ncache, seed, share=True):
    rng = np.random.default_rng(seed)
    s = rng.permutation(ncache)[:B].astype(np.int32)
    s[B // 3] = -1                       # inactive: below the pool
    s[B // 2] = ncache                   # inactive: past the pool
    if share:
        s[-1] = s[0]                     # two rows read one cache row
    return s


CASES = [  # (B, Hq, Hkv, Smax, d, dtype, ncache)
    (8, 12, 2, 2048, 128, torch.bfloat16, 20),
    (6, 32, 8, 700, 64, torch.bfloat16, 9),
    (5, 4, 1, 333, 32, torch.bfloat16, 7),
    (7, 8, 2, 300, 64, torch.float32, 11),
    (6, 40, 1, 500, 128, torch.bfloat16, 8),    # g = 40: two 16-head column blocks per wave
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_slots_plain_decode(case):
    B, Hq, Hkv, Smax, d, dtype, ncache = CASES[case]
    kc, vc = _pool(ncache, Hkv, Smax, d, dtype, 50 + case)
    q = random_tensor((B, Hq, d), 60 + case, dtype)
    slots = _slots(B, ncache, 70 + case)
    lens = np.random.default_rng(80 + case).integers(0, Smax + 1, B).astype(np.int32)
    lens[0], lens[1] = Smax, 0
    out = attn_decode_slots(q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(slots).to(DEV),
                            torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    ref = oracle.attn_decode_slots(q, kc, vc, slots, lens)
    err = float(np.max(np.abs(got - ref)))
    print(f"slots decode B{B} Hq{Hq} Hkv{Hkv} Smax{Smax} d{d} {dtype} pool {ncache}: "
          f"max abs error {err:.3g}")
    assert err <= TOL[dtype]
    for b in range(B):
        if not 0 <= slots[b] < ncache or lens[b] == 0:
            assert np.all(got[b] == 0), f"row {b} should be zero"


@pytest.mark.parametrize("case", range(len(CASES)))
def test_slots_append(case):
    B, Hq, Hkv, Smax, d, dtype, ncache = CASES[case]
    kc, vc = _pool(ncache, Hkv, Smax, d, dtype, 150 + case)
    q = random_tensor((B, Hq, d), 160 + case, dtype)
    kn = random_tensor((B, Hkv, d), 161 + case, dtype)
    vn = random_tensor((B, Hkv, d), 162 + case, dtype)
    slots = _slots(B, ncache, 170 + case, share=False)
    pos = np.random.default_rng(180 + case).integers(0, Smax, B).astype(np.int32)
    pos[0] = Smax - 1
    kd, vd = kc.to(DEV), vc.to(DEV)
    out = attn_decode_slots(q.to(DEV), kd, vd, torch.from_numpy(slots).to(DEV),
                            torch.from_numpy(pos).to(DEV), k_new=kn.to(DEV), v_new=vn.to(DEV))
    torch.cuda.synchronize()
    ref, kref, vref = oracle.attn_decode_slots(q, kc, vc, slots, pos, k_new=kn, v_new=vn)
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    print(f"slots append B{B} Hq{Hq} Hkv{Hkv} Smax{Smax} d{d} {dtype}: max abs error {err:.3g}")
    assert err <= TOL[dtype]
    assert np.array_equal(kd.cpu().double().numpy(), kref)
    assert np.array_equal(vd.cpu().double().numpy(), vref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_identity_table_is_the_plain_batch(dtype):
    B, Hq, Hkv, Smax, d = 8, 12, 2, 1000, 128
    kc, vc = (t.to(DEV) for t in _pool(B, Hkv, Smax, d, dtype, 200))
    q = random_tensor((B, Hq, d), 201, dtype).to(DEV)
    lens = torch.tensor([1000, 0, 17, 512, 999, 1, 640, 33], dtype=torch.int32, device=DEV)
    ident = torch.arange(B, dtype=torch.int32, device=DEV)
    assert torch.equal(attn_decode_slots(q, kc, vc, ident, lens), attn_decode(q, kc, vc, lens))
    kn = random_tensor((B, Hkv, d), 202, dtype).to(DEV)
    vn = random_tensor((B, Hkv, d), 203, dtype).to(DEV)
    pos = torch.tensor([999, -1, 16, 511, 998, 0, 639, 32], dtype=torch.int32, device=DEV)
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    a = attn_decode_slots(q, k1, v1, ident, pos, k_new=kn, v_new=vn)
    b = attn_decode_append(q, kn, vn, k2, v2, pos)
    assert torch.equal(a, b) and torch.equal(k1, k2) and torch.equal(v1, v2)


def test_relabelled_pool_gives_the_same_bits():
    ncache, B, Hq, Hkv, Smax, d = 10, 6, 12, 2, 800, 128
    kc, vc = _pool(ncache, Hkv, Smax, d, torch.bfloat16, 300)
    q = random_tensor((B, Hq, d), 301, torch.bfloat16).to(DEV)
    slots = np.array([3, 7, 0, 9, 3, 5], dtype=np.int32)
    lens = torch.tensor([800, 300, 1, 77, 650, 512], dtype=torch.int32, device=DEV)
    o1 = attn_decode_slots(q, kc.to(DEV), vc.to(DEV), torch.from_numpy(slots).to(DEV), lens)
    perm = torch.from_numpy(np.random.default_rng(302).permutation(ncache))
    kp, vp = torch.empty_like(kc), torch.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    s2 = perm.numpy()[slots].astype(np.int32)
    o2 = attn_decode_slots(q, kp.to(DEV), vp.to(DEV), torch.from_numpy(s2).to(DEV), lens)
    assert torch.equal(o1, o2)


def test_large_pool():
    """40 active rows of a 64-row pool (Hq 16, Hkv 4, Smax 2048, d 128, bf16),
    every element against the oracle."""
    ncache, B, Hq, Hkv, Smax, d = 64, 40, 16, 4, 2048, 128
    kc, vc = _pool(ncache, Hkv, Smax, d, torch.bfloat16, 400)
    q = random_tensor((B, Hq, d), 401, torch.bfloat16)
    slots = np.random.default_rng(402).permutation(ncache)[:B].astype(np.int32)
    lens = np.random.default_rng(403).integers(1, Smax + 1, B).astype(np.int32)
    out = attn_decode_slots(q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(slots).to(DEV),
                            torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attn_decode_slots(q, kc, vc, slots, lens)
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    print(f"slots decode large pool: max abs error {err:.3g}")
    assert err <= 2e-2
