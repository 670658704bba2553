"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Bar: max |O_gpu - O_oracle| <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs, over every compared element, with the oracle fed the exact same
(rounded) inputs.  The named workloads run at full size: compared in full
where the oracle takes seconds, on sampled rows plus size-independent
properties where it does not.  Small cases span several tiles, ragged tails,
every head-grouping mode and the method's degenerate cases.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import attn_decode, attn_fwd
from mqa_flashattention_amd.workloads import (WORKLOADS, DecodeShape, FwdShape, decode_inputs,
                                              fwd_inputs, random_tensor)

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().to("cpu").double().numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def _fwd_gpu(q, k, v, **kw):
    out = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return out.cpu()


def _check_fwd(s: FwdShape, seed: int = 0, rows: int | None = None):
    q, k, v = fwd_inputs(s, seed)
    out = _fwd_gpu(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    if rows is None:
        ref = oracle.attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
        err = _err(out, ref)
    else:
        total = s.B * s.Hq * s.Nq
        rng = np.random.default_rng(seed + 17)
        ids = np.unique(np.concatenate([rng.integers(0, total, rows),
                                        [0, s.Nq - 1, total - s.Nq, total - 1]]))
        ref = oracle.attn_fwd_rows(q, k, v, ids, causal=s.causal, q_offset=s.q_offset,
                                   scale=s.scale)
        err = _err(out.reshape(-1, s.d)[torch.from_numpy(ids)], ref)
    assert err <= TOL[s.dtype], f"{s}: max abs error {err}"
    return q, k, v, out


# ---------------------------------------------------------------- named workloads

def test_tiny_gqa_fp32():
    _check_fwd(WORKLOADS["tiny_gqa_f32"].fwd[0])


def test_llama3_8b_causal_prefill_full():
    _check_fwd(WORKLOADS["llama3_8b_prefill"].fwd[0])


@pytest.mark.parametrize("variant", [0, 1, 2], ids=["mha_hkv16", "gqa_hkv4", "mqa_hkv1"])
def test_mha_gqa_mqa_sweep_full(variant):
    """Every element of each variant against the oracle (about 275 GFLOP of
    fp64 per variant on the host), then GQA = MHA with K/V heads repeated on
    the GPU, bit for bit up to the tolerance."""
    s = WORKLOADS["mha_gqa_mqa_sweep"].fwd[variant]
    q, k, v, out = _check_fwd(s)
    if s.Hkv < s.Hq:
        g = s.Hq // s.Hkv
        mha = _fwd_gpu(q, k.repeat_interleave(g, 1).contiguous(),
                       v.repeat_interleave(g, 1).contiguous(), scale=s.scale)
        diff = float((mha.double() - out.double()).abs().max())
        assert diff <= TOL[s.dtype], f"GQA vs replicated MHA differ by {diff}"


def test_chunked_prefill_full():
    _check_fwd(WORKLOADS["chunked_prefill_4k"].fwd[0])


def test_kv_decode_full():
    s = WORKLOADS["kv_decode_b8"].decode
    q, kc, vc, lens = decode_inputs(s, 0)
    out = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=s.scale)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(q, kc, vc, lens, scale=s.scale)
    err = _err(out, ref)
    assert err <= TOL[s.dtype], f"decode max abs error {err}"
    # Slots at or past each row's length are never read: NaN there changes nothing.
    kp, vp = kc.clone(), vc.clone()
    for b in range(s.B):
        kp[b, :, int(lens[b]):] = float("nan")
        vp[b, :, int(lens[b]):] = float("nan")
    out2 = attn_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), lens.to(DEV), scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out2.cpu())


# ---------------------------------------------------------------- small-case matrix
# MHA (g=1), GQA (g=2, 4, 6) and MQA (Hkv=1) as in the "Kernel 9" test matrix
# of the BootstrapAI log, over head dims, ragged lengths and causal offsets.

MODES = [(4, 4), (4, 2), (8, 2), (12, 2), (8, 1)]
LENGTHS = [(1, 1), (17, 17), (63, 65), (65, 63), (129, 129), (40, 200), (200, 40)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("hq,hkv", MODES)
def test_small_matrix(dtype, d, hq, hkv):
    seed = 1000 + d + 10 * hq + hkv
    for n, (nq, nk) in enumerate(LENGTHS):
        for causal, off in ((False, 0), (True, 0), (True, max(0, nk - nq)), (True, 7)):
            s = FwdShape(2, hq, hkv, nq, nk, d, causal, off, dtype)
            _check_fwd(s, seed + n)


@pytest.mark.parametrize("g", [40, 160])
def test_large_groups(g):
    """More query heads per K/V head than one unit (128 columns) or one decode
    wave (32 columns) holds."""
    s = FwdShape(1, g, 1, 37, 70, 64, True, 5)
    _check_fwd(s, 5)
    ds = DecodeShape(2, g, 1, 90, 64, 1, 90)
    q, kc, vc, lens = decode_inputs(ds, 6)
    out = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV))
    torch.cuda.synchronize()
    assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= TOL[ds.dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_lengths(dtype, d):
    B, Hq, Hkv, Smax = 9, 6, 2, 300
    q = random_tensor((B, Hq, d), 1, dtype)
    kc = random_tensor((B, Hkv, Smax, d), 2, dtype)
    vc = random_tensor((B, Hkv, Smax, d), 3, dtype)
    lens = torch.tensor([1, 31, 32, 33, 64, 65, 299, 300, 150], dtype=torch.int32)
    out = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV))
    torch.cuda.synchronize()
    assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= TOL[dtype]


def test_decode_empty_and_overlong_rows():
    """n = clamp(seqlens, 0, Smax): zero/negative lengths give zero rows,
    lengths beyond the capacity read the whole cache."""
    B, Hq, Hkv, Smax, d = 4, 4, 1, 70, 128
    q = random_tensor((B, Hq, d), 11, torch.bfloat16)
    kc = random_tensor((B, Hkv, Smax, d), 12, torch.bfloat16)
    vc = random_tensor((B, Hkv, Smax, d), 13, torch.bfloat16)
    lens = torch.tensor([0, -5, 70, 1000], dtype=torch.int32)
    out = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)).cpu()
    torch.cuda.synchronize()
    assert torch.all(out[:2] == 0)
    assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= 2e-2


def test_decode_matches_single_query_forward():
    """Decode of row b equals the forward pass with one query over its n keys."""
    s = DecodeShape(3, 8, 2, 257, 128, 1, 257)
    q, kc, vc, lens = decode_inputs(s, 21)
    dec = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)).cpu().double()
    for b in range(s.B):
        n = int(lens[b])
        f = _fwd_gpu(q[b:b + 1, :, None, :].contiguous(), kc[b:b + 1, :, :n].contiguous(),
                     vc[b:b + 1, :, :n].contiguous())
        assert float((f[0, :, 0].double() - dec[b]).abs().max()) <= 2e-2


# Decode shapes large enough for splits of several 32-token tiles and many
# splits per row, with lengths on and around tile and split boundaries.
@pytest.mark.parametrize("B,Hq,Hkv,Smax,d,dtype", [
    (24, 12, 2, 2048, 128, torch.bfloat16),
    (64, 8, 1, 4096, 64, torch.bfloat16),
    (16, 40, 1, 2048, 32, torch.float32),     # two 32-head column blocks
], ids=["b24_d128", "b64_d64", "b16_g40_f32"])
def test_decode_multi_tile_splits(B, Hq, Hkv, Smax, d, dtype):
    g = torch.Generator().manual_seed(B + Smax + d)
    special = [1, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, Smax - 1, Smax]
    lens = torch.randint(1, Smax + 1, (B,), generator=g, dtype=torch.int32)
    lens[:len(special)] = torch.tensor(special[:B], dtype=torch.int32)
    q = random_tensor((B, Hq, d), 91, dtype)
    kc = random_tensor((B, Hkv, Smax, d), 92, dtype)
    vc = random_tensor((B, Hkv, Smax, d), 93, dtype)
    out = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV))
    torch.cuda.synchronize()
    assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= TOL[dtype]


# Larger batches: several parts per row and several rounds of workgroups.
# Empty rows (length 0 or negative) at the start, in the middle and at the
# end; MHA, GQA and two column groups per K/V head; slots past each length
# poisoned with NaN.
LARGE_DECODE_SHAPES = [(40, 12, 2, 1500, 128), (20, 40, 1, 2000, 64), (33, 8, 8, 1200, 32),
                 (128, 12, 2, 2048, 128)]


@pytest.mark.parametrize("B,Hq,Hkv,Smax,d", LARGE_DECODE_SHAPES,
                         ids=["gqa6_d128", "g40_d64", "mha_d32", "b128_d128"])
def test_decode_large_batches(B, Hq, Hkv, Smax, d):
    g = torch.Generator().manual_seed(B * Smax + d)
    lens = torch.randint(1, Smax + 1, (B,), generator=g, dtype=torch.int32)
    special = [0, 0, 1, 31, 32, 33, Smax, Smax + 5, -3]
    lens[:len(special)] = torch.tensor(special, dtype=torch.int32)
    lens[B // 2] = 0
    lens[B - 1] = 0
    q = random_tensor((B, Hq, d), 61, torch.bfloat16)
    kc = random_tensor((B, Hkv, Smax, d), 62, torch.bfloat16)
    vc = random_tensor((B, Hkv, Smax, d), 63, torch.bfloat16)
    kp, vp = kc.clone(), vc.clone()
    for b in range(B):
        n = max(0, min(int(lens[b]), Smax))
        kp[b, :, n:] = float("nan")
        vp[b, :, n:] = float("nan")
    out = attn_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), lens.to(DEV))
    torch.cuda.synchronize()
    assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= 2e-2
    empty = [b for b in range(B) if int(lens[b]) <= 0]
    assert torch.all(out.cpu()[empty] == 0)


def test_decode_across_sizes_and_streams():
    """Calls of growing and shrinking row counts on one stream, then the same
    inputs on two streams: every output equals the first call's, bit for bit."""
    cases = []
    for B, Smax in ((2, 600), (40, 1500), (3, 600)):
        s = DecodeShape(B, 12, 2, Smax, 128, 1, Smax)
        q, kc, vc, lens = decode_inputs(s, 30 + B)
        dev = tuple(t.to(DEV) for t in (q, kc, vc, lens))
        out = attn_decode(*dev)
        torch.cuda.synchronize()
        assert _err(out, oracle.attn_decode(q, kc, vc, lens)) <= 2e-2
        cases.append((dev, out))
    for dev, out in cases:
        assert torch.equal(attn_decode(*dev), out)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = []
    for st in (s1, s2):
        with torch.cuda.stream(st):
            res.append([attn_decode(*dev) for dev, _ in cases for _ in range(2)])
    torch.cuda.synchronize()
    for group in res:
        for i, o in enumerate(group):
            assert torch.equal(o, cases[i // 2][1])


def test_decode_bitwise_deterministic_many_splits():
    s = DecodeShape(24, 12, 2, 2048, 128, 1, 2048)
    dq, dk, dv, dl = (t.to(DEV) for t in decode_inputs(s, 5))
    d1 = attn_decode(dq, dk, dv, dl)
    for _ in range(20):
        assert torch.equal(d1, attn_decode(dq, dk, dv, dl))
    torch.cuda.synchronize()


# ---------------------------------------------------------------- properties / edge cases

def test_causal_row0_and_constant_v_exact():
    """bf16: causal row 0 returns V[0] bit-exactly; a constant V comes back exactly."""
    s = FwdShape(1, 8, 2, 130, 130, 128, True, 0)
    q, k, v = fwd_inputs(s, 3)
    out = _fwd_gpu(q, k, v, causal=True)
    for h in range(8):
        assert torch.equal(out[0, h, 0], v[0, h // 4, 0])
    vconst = torch.full_like(v, -1.25)
    out = _fwd_gpu(q, k, vconst, causal=True)
    assert torch.all(out == -1.25)


def test_chunked_equals_rows_of_full_pass():
    N, off, n = 700, 450, 130
    s = FwdShape(1, 8, 2, N, N, 64, True, 0)
    q, k, v = fwd_inputs(s, 8)
    full = _fwd_gpu(q, k, v, causal=True)
    part = _fwd_gpu(q[:, :, off:off + n].contiguous(), k, v, causal=True, q_offset=off)
    assert float((full[:, :, off:off + n].double() - part.double()).abs().max()) <= 2e-2


@pytest.mark.parametrize("scale", [0.0, -0.2, 3.0])
def test_unusual_scales(scale):
    s = FwdShape(1, 4, 2, 70, 90, 64, True, 20)
    q, k, v = fwd_inputs(s, 9)
    out = _fwd_gpu(q, k, v, causal=True, q_offset=20, scale=scale)
    ref = oracle.attn_fwd(q, k, v, causal=True, q_offset=20, scale=scale)
    assert _err(out, ref) <= 2e-2


def test_output_guard_bands_untouched():
    s = FwdShape(2, 4, 2, 77, 77, 128, True, 0)
    q, k, v = fwd_inputs(s, 10)
    buf = torch.full((4, 4, 77, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[1:3]
    attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[0] == 7.0) and torch.all(buf[3] == 7.0)
    ref = oracle.attn_fwd(q, k, v, causal=True)
    assert _err(out, ref) <= 2e-2


@pytest.mark.parametrize("name,variant", [("llama3_8b_prefill", 0), ("mha_gqa_mqa_sweep", 1),
                                          ("chunked_prefill_4k", 0)],
                         ids=["pair", "persistent_atomic", "quad"])
def test_bitwise_deterministic_runs(name, variant):
    """Each output's arithmetic order is fixed -- the persistent schedule's
    atomics only change which workgroup runs a unit, and every merge runs in
    a fixed order -- so 20 repeated runs agree bit for bit, on each schedule
    the named workloads use."""
    s = WORKLOADS[name].fwd[variant]
    q, k, v = (t.to(DEV) for t in fwd_inputs(s, 0))
    first = attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    for _ in range(20):
        again = attn_fwd(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
        assert torch.equal(first, again)
    torch.cuda.synchronize()


def test_llama_layer_batch4_persistent_causal():
    """The LLaMA-3-8B prefill layer at batch 4 (2048 units of 128 columns, more
    than two per resident workgroup) runs on the persistent schedule -- the
    per-XCD atomic queues, heaviest position blocks first, stealing.  Every
    element is compared with the oracle, and 20 more runs agree bit for bit."""
    s = FwdShape(4, 32, 8, 2048, 2048, 128, True, 0)
    q, k, v, out = _check_fwd(s, 7)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    first = out.to(DEV)
    for _ in range(20):
        assert torch.equal(first, attn_fwd(qd, kd, vd, causal=True, scale=s.scale))
    torch.cuda.synchronize()


def test_decode_bitwise_deterministic_runs():
    ds = WORKLOADS["kv_decode_b8"].decode
    dq, dk, dv, dl = (t.to(DEV) for t in decode_inputs(ds, 0))
    d1 = attn_decode(dq, dk, dv, dl)
    for _ in range(20):
        assert torch.equal(d1, attn_decode(dq, dk, dv, dl))
    torch.cuda.synchronize()


@pytest.mark.parametrize("n", [127, 1000])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_ragged_tails(n, causal):
    """Sequence lengths one short of a tile multiple and far from one."""
    for d, dtype in ((128, torch.bfloat16), (64, torch.bfloat16), (32, torch.float32)):
        s = FwdShape(1, 8, 2, n, n, d, causal, 0, dtype)
        _check_fwd(s, 40 + d)


def test_two_streams_keep_separate_schedulers():
    s = FwdShape(1, 8, 2, 300, 300, 64, True, 0)
    q, k, v = (t.to(DEV) for t in fwd_inputs(s, 12))
    ref = attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for st in (s1, s2):
        with torch.cuda.stream(st):
            outs.append([attn_fwd(q, k, v, causal=True) for _ in range(3)])
    torch.cuda.synchronize()
    for group in outs:
        for o in group:
            assert torch.equal(o, ref)


# ---------------------------------------------------------------- key-split units
# Launches with few units cut each slice's key tiles into equal chunks, one
# per workgroup; units that a chunk boundary cuts are merged from their pieces.

SPLIT_SHAPES = [
    # MQA, 8 units of 256 tiles: every unit is cut into many pieces
    FwdShape(1, 8, 1, 128, 8192, 128, False, 0),
    # MHA causal with an offset: parts where some query rows see no key
    FwdShape(1, 2, 2, 700, 737, 64, True, 37),
    # fp32 chunk at the end of a long cache
    FwdShape(2, 4, 1, 64, 2000, 32, True, 1936, torch.float32),
    # GQA causal prefill, one sequence
    FwdShape(1, 16, 2, 1500, 1500, 128, True, 0),
]


@pytest.mark.parametrize("s", SPLIT_SHAPES, ids=["mqa_long_keys", "mha_causal_offset",
                                                 "f32_chunk", "gqa_causal"])
def test_key_split_parity_and_determinism(s):
    q, k, v, out = _check_fwd(s, 31)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for _ in range(5):
        again = attn_fwd(qd, kd, vd, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
        assert torch.equal(again.cpu(), out)


def test_key_split_workspace_regrows_between_sizes():
    """Launches with cut units, of growing and shrinking sizes, on one stream."""
    shapes = [FwdShape(1, 4, 1, 32, 2000, 64, False, 0),
              FwdShape(1, 8, 1, 128, 8192, 128, False, 0),
              FwdShape(1, 4, 1, 32, 2000, 64, False, 0)]
    for n, s in enumerate(shapes):
        _check_fwd(s, 40 + n)


# ---------------------------------------------------------------- pair schedule
# Causal launches with at least one heavy/light unit pair per CU run one pair
# per 8-wave workgroup whose halves split each unit's keys (the LLaMA-shaped
# prefill above is one); these cover an odd number of position blocks (the
# middle unit runs alone), a chunk at an offset, and fp32.

PAIR_SHAPES = [
    FwdShape(2, 8, 8, 4100, 4100, 128, True, 0),
    FwdShape(8, 32, 8, 256, 3000, 128, True, 2744),
    FwdShape(4, 16, 2, 1030, 1030, 64, True, 0, torch.float32),
]


@pytest.mark.parametrize("s", PAIR_SHAPES, ids=["mha_odd_blocks", "gqa_chunk_offset", "f32_gqa"])
def test_pair_schedule_full(s):
    q, k, v, out = _check_fwd(s, 51)
    again = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, q_offset=s.q_offset,
                     scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(again.cpu(), out)


# ---------------------------------------------------------------- random shapes
# Seeded random shapes against the oracle, every element compared: small ones,
# and larger ones sized so the persistent (many units), pair (causal, at least
# one unit pair per CU) and balanced (few units) schedules all run.

# Shapes with fewer 128-column units than CUs but 192-256 64-column units of
# >= 8 key tiles: on a 256-CU MI355X they run on the quad schedule (one
# 8-wave workgroup per 64-column unit, keys split four ways, merged in LDS).
QUAD_SHAPES = [
    FwdShape(2, 32, 8, 256, 1024, 128, True, 768),
    FwdShape(2, 32, 8, 256, 600, 64, True, 344, torch.float32),
    FwdShape(1, 32, 1, 400, 600, 64, False, 0),
    FwdShape(1, 160, 1, 70, 570, 64, True, 500),
    FwdShape(2, 16, 4, 512, 1024, 32, True, 512),
    # a ragged last key tile (1000 = 31 * 32 + 8) on the direct K loads
    FwdShape(2, 32, 8, 256, 1000, 128, True, 744),
]


@pytest.mark.parametrize("s", QUAD_SHAPES, ids=["gqa_d128_offset", "f32_d64_offset", "mqa_g32",
                                                "g160_three_head_blocks", "d32_offset",
                                                "gqa_d128_ragged_keys"])
def test_quad_schedule(s):
    q, k, v, out = _check_fwd(s, 13)
    again = _fwd_gpu(q, k, v, causal=s.causal, q_offset=s.q_offset, scale=s.scale)
    assert torch.equal(out, again), "quad schedule not bitwise reproducible"


def _random_shapes():
    rng = np.random.default_rng(2024)
    shapes = []
    for _ in range(24):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        d = int(rng.choice([32, 64, 128]))
        nq = int(rng.integers(1, 300))
        nk = int(rng.integers(1, 400))
        causal = bool(rng.random() < 0.6)
        off = int(rng.integers(0, nk)) if causal else 0
        dt = torch.float32 if rng.random() < 0.3 else torch.bfloat16
        shapes.append((FwdShape(int(rng.integers(1, 4)), hkv * g, hkv, nq, nk, d, causal, off, dt),
                       None))
    # many units: persistent schedule
    shapes.append((FwdShape(2, 32, 8, 2100, 2100, 128, True, 0), None))
    shapes.append((FwdShape(6, 24, 4, 1500, 1700, 64, False, 0), None))
    shapes.append((FwdShape(4, 40, 8, 1100, 1300, 128, True, 200, torch.float32), None))
    # non-causal d = 128 with more than two units per resident workgroup: persistent
    # schedule with K loaded straight into LDS, last key tile ragged (2300 = 71 * 32 + 28)
    shapes.append((FwdShape(2, 32, 8, 2200, 2300, 128, False, 0), None))
    # causal, one pair per CU or more: pair schedule
    shapes.append((FwdShape(1, 48, 12, 2000, 2000, 128, True, 0), None))
    shapes.append((FwdShape(2, 40, 8, 1100, 1300, 128, True, 200, torch.float32), None))
    # few units, cut chunks: balanced schedule
    shapes.append((FwdShape(4, 8, 2, 1900, 2500, 64, True, 600), None))
    return shapes


RANDOM_SHAPES = _random_shapes()


@pytest.mark.parametrize("idx", range(len(RANDOM_SHAPES)))
def test_random_shapes(idx):
    s, rows = RANDOM_SHAPES[idx]
    _check_fwd(s, 300 + idx, rows=rows)


# ---------------------------------------------------------------- HIP graph capture
def test_decode_graph_replay_matches_eager():
    """Decode calls captured in a HIP graph (caller-provided workspace: the
    decode path allocates nothing and issues no memset) replay to the eager
    results, bit for bit, on every replay, with eager work and
    synchronisations between the replays."""
    s = WORKLOADS["kv_decode_b8"].decode
    cases = []
    for seed in (0, 1, 2):
        q, kc, vc, lens = (t.to(DEV) for t in decode_inputs(s, seed))
        cases.append((q, kc, vc, lens))
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    eager = [attn_decode(*c, workspace=ws).clone() for c in cases]
    outs = [torch.empty_like(c[0]) for c in cases]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c, o in zip(cases, outs):
            attn_decode(*c, out=o, workspace=ws)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager call"
        # eager work between replays, on the same workspace
        assert torch.equal(attn_decode(*cases[rep % 3], workspace=ws), eager[rep % 3])
        torch.cuda.synchronize()
