"""GPU parity at the size limits: tensors past 4 GiB (offsets that overflow
32 bits), the largest decode batch the grid takes, and a packed batch of
thousands of sequences.  Inputs are drawn on the GPU from seeded generators
(N(0,1), rounded to bf16); rows are sampled -- the first and last ones of
the first and last batches and heads included -- and each is compared with
the oracle on its own batch's tensors, at the forward's bar (2e-2).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_decode, attn_fwd, attn_fwd_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _randn(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def test_prefill_tensors_past_4gib():
    """B 528, Hq 32, Hkv 8, N 1024, d 128, causal: Q and O are 4.4 GB each."""
    B, Hq, Hkv, N, d = 528, 32, 8, 1024, 128
    q, k, v = _randn((B, Hq, N, d), 1), _randn((B, Hkv, N, d), 2), _randn((B, Hkv, N, d), 3)
    assert q.numel() * 2 > 2 ** 32
    o = attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    worst = 0.0
    for b in [0, 1, 255, B - 2, B - 1]:
        rows = np.unique(np.concatenate([[0, N - 1, (Hq - 1) * N, Hq * N - 1],
                                         rng.integers(0, Hq * N, 12)]))
        ref = oracle.attn_fwd_rows(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), rows,
                                   causal=True)
        got = o[b].reshape(-1, d)[torch.from_numpy(rows).to(DEV)].cpu().double().numpy()
        worst = max(worst, float(np.max(np.abs(got - ref))))
    print(f"prefill past 4 GiB: max abs error {worst:.3g}")
    assert worst <= 2e-2


def test_decode_largest_batch():
    """B = 65535 rows (the grid's limit), Hq 4, Hkv 1, Smax 64, d 32, lengths
    U[0, 64]."""
    B, Hq, Hkv, S, d = 65535, 4, 1, 64, 32
    q, kc, vc = _randn((B, Hq, d), 5), _randn((B, Hkv, S, d), 6), _randn((B, Hkv, S, d), 7)
    lens_h = torch.from_numpy(np.random.default_rng(8).integers(0, S + 1, B).astype(np.int32))
    o = attn_decode(q, kc, vc, lens_h.to(DEV))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, B // 2, B - 2, B - 1],
                                     np.random.default_rng(9).integers(0, B, 60)]))
    idx = torch.from_numpy(rows).to(DEV)
    ref = oracle.attn_decode(q[idx].cpu(), kc[idx].cpu(), vc[idx].cpu(), lens_h[rows])
    err = float(np.max(np.abs(o[idx].cpu().double().numpy() - ref)))
    print(f"decode B=65535: max abs error {err:.3g}")
    assert err <= 2e-2
    empty = torch.from_numpy(np.nonzero(lens_h.numpy() == 0)[0]).to(DEV)
    assert empty.numel() > 0 and torch.count_nonzero(o[empty]) == 0


def test_varlen_thousands_of_sequences():
    """20000 causal sequences of 1..40 queries over 0..60 keys in one launch."""
    rng = np.random.default_rng(10)
    nseq, Hq, Hkv, d = 20000, 8, 2, 64
    lq = rng.integers(1, 41, nseq)
    lk = rng.integers(0, 61, nseq)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _randn((int(cq[-1]), Hq, d), 11), _randn((int(ck[-1]), Hkv, d), 12), \
        _randn((int(ck[-1]), Hkv, d), 13)
    o = attn_fwd_varlen(q, k, v, torch.from_numpy(cq).to(DEV), torch.from_numpy(ck).to(DEV),
                        int(lq.max()), causal=True)
    torch.cuda.synchronize()
    worst = 0.0
    for s in np.unique(np.concatenate([[0, 1, nseq - 1], rng.integers(0, nseq, 40)])):
        q0, q1, k0, k1 = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
        ref = oracle.attn_fwd_varlen(q[q0:q1].cpu(), k[k0:k1].cpu(), v[k0:k1].cpu(),
                                     np.array([0, q1 - q0]), np.array([0, k1 - k0]), causal=True)
        worst = max(worst, float(np.max(np.abs(o[q0:q1].cpu().double().numpy() - ref))))
    print(f"varlen 20000 sequences: max abs error {worst:.3g}")
    assert worst <= 2e-2
