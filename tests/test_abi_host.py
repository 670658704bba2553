"""CPU tests of the C ABI: the library loads, exports what include/gqa_attn.h
declares, and rejects every invalid argument on the host before any HIP call.

No kernel is launched: every call here fails validation (or, with no GPU
visible, the device check), so the pointers passed are never dereferenced.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

from mqa_flashattention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

OK, NULLP, SHAPE, GROUP, UNSUP, WS, NODEV, HIP = range(8)
BF16, F32 = 1, 0
# Distinct, 16-byte-aligned stand-ins for device pointers (never dereferenced).
P = [ctypes.c_void_p(0x10000 * (n + 1)) for n in range(8)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIBRARY], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, f"not exported: {missing}"
    for f in declared_functions():
        assert hasattr(binding.lib, f)


def test_library_embeds_gfx950_code_only():
    blob = open(binding.LIBRARY, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-f]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_status_strings():
    for code in range(8):
        s = binding.lib.gqa_status_string(code)
        assert s and isinstance(s, bytes)
    assert binding.lib.gqa_status_string(99) == b"unknown status"


def fwd(q=P[0], k=P[1], v=P[2], o=P[3], B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=32, causal=0,
        q_offset=0, scale=0.17, dtype=BF16, stream=None):
    return binding.lib.gqa_attn_fwd(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, causal, q_offset,
                                    ctypes.c_float(scale), dtype, stream)


def dec(q=P[0], kc=P[1], vc=P[2], sl=P[4], o=P[3], B=8, Hq=12, Hkv=2, Smax=2048, d=128,
        scale=0.09, dtype=BF16, ws=P[5], ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = binding.decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    return binding.lib.gqa_attn_decode(q, kc, vc, sl, o, B, Hq, Hkv, Smax, d,
                                       ctypes.c_float(scale), dtype, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(k=None), NULLP), (dict(v=None), NULLP), (dict(o=None), NULLP),
    (dict(B=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=-1), SHAPE), (dict(Nq=0), SHAPE),
    (dict(Nk=0), SHAPE), (dict(d=0), SHAPE), (dict(causal=1, q_offset=-1), SHAPE),
    (dict(Nk=2 ** 30, d=32), SHAPE),
    (dict(Hq=6, Hkv=4), GROUP), (dict(Hq=3, Hkv=2), GROUP),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(d=16), UNSUP),
    (dict(dtype=2), UNSUP), (dict(dtype=-1), UNSUP),
    (dict(scale=float("inf")), UNSUP), (dict(scale=float("nan")), UNSUP),
    (dict(q=ctypes.c_void_p(0x10008)), UNSUP), (dict(o=ctypes.c_void_p(0x40002)), UNSUP),
])
def test_fwd_rejects_invalid_arguments(kw, code):
    assert fwd(**kw) == code
    assert binding.lib.gqa_last_error_string()


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(kc=None), NULLP), (dict(vc=None), NULLP),
    (dict(sl=None), NULLP), (dict(o=None), NULLP),
    (dict(B=0), SHAPE), (dict(Smax=0), SHAPE), (dict(Hkv=0), SHAPE),
    (dict(Smax=2 ** 25, d=128), SHAPE),
    (dict(Hq=12, Hkv=5), GROUP),
    (dict(d=80), UNSUP), (dict(dtype=7), UNSUP), (dict(scale=float("-inf")), UNSUP),
    (dict(kc=ctypes.c_void_p(0x20004)), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS), (dict(ws=ctypes.c_void_p(0x60008)), WS),
])
def test_decode_rejects_invalid_arguments(kw, code):
    assert dec(**kw) == code
    assert binding.lib.gqa_last_error_string()


def dec_na(q=P[0], kc=P[1], vc=P[2], sl=P[4], o=P[3], B=8, Hq=12, Hkv=2, Smax=2048, d=128,
           scale=0.09, dtype=BF16, stream=None):
    return binding.lib.gqa_attn_decode_noalloc(q, kc, vc, sl, o, B, Hq, Hkv, Smax, d,
                                               ctypes.c_float(scale), dtype, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(kc=None), NULLP), (dict(vc=None), NULLP),
    (dict(sl=None), NULLP), (dict(o=None), NULLP),
    (dict(B=0), SHAPE), (dict(Smax=0), SHAPE), (dict(Smax=2 ** 25, d=128), SHAPE),
    (dict(Hq=12, Hkv=5), GROUP), (dict(d=80), UNSUP), (dict(dtype=7), UNSUP),
    (dict(kc=ctypes.c_void_p(0x20004)), UNSUP),
    # split records beyond the static scratch
    (dict(B=64, Hq=32, Hkv=8, Smax=32768), WS),
])
def test_decode_noalloc_rejects_invalid_arguments(kw, code):
    assert dec_na(**kw) == code
    assert binding.lib.gqa_last_error_string()


def test_decode_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GQA_DECODE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "limit not found in the header"
    assert int(m.group(1)) << int(m.group(2)) == binding.DECODE_NOALLOC_SCRATCH_BYTES
    # the batch-8 decode workload fits
    assert binding.decode_workspace_bytes(8, 12, 2, 2048, 128) <= \
        binding.DECODE_NOALLOC_SCRATCH_BYTES


def fwd_s(q=P[0], k=P[1], v=P[2], o=P[3], B=2, Hq=8, Hkv=2, Nq=64, Nk=96, d=64, qs=None,
          kvs=None, causal=1, q_offset=0, scale=0.17, dtype=BF16, stream=None):
    """Strided forward; default strides are BTHD (token-major)."""
    I3 = ctypes.c_int64 * 3
    qs = I3(*(qs if qs is not None else (Nq * Hq * d, d, Hq * d)))
    kvs = I3(*(kvs if kvs is not None else (Nk * Hkv * d, d, Hkv * d)))
    return binding.lib.gqa_attn_fwd_strided(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, qs, kvs, causal,
                                            q_offset, ctypes.c_float(scale), dtype, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(o=None), NULLP),
    (dict(qs=(-1, 64, 512)), SHAPE), (dict(kvs=(0, 64, -128)), SHAPE),
    (dict(qs=(64 * 8 * 64, 64, 8 * 64 + 4)), UNSUP),   # token stride not 16-byte aligned
    (dict(kvs=(3, 64, 128)), UNSUP),                    # batch stride not 16-byte aligned
    (dict(qs=(64 * 8 * 64, 64, 32)), SHAPE),            # output rows overlap (token < d)
    (dict(qs=(0, 64, 512)), SHAPE),                     # batches alias in the output
    (dict(qs=(64 * 8 * 64, 0, 512)), SHAPE),            # heads alias in the output
    (dict(kvs=(0, 64, 2 ** 24)), SHAPE),                # K/V token stride too large
    (dict(Hq=6, Hkv=4), GROUP), (dict(d=48), UNSUP), (dict(B=0), SHAPE),
    (dict(q=ctypes.c_void_p(0x10008)), UNSUP),
])
def test_fwd_strided_rejects_invalid_arguments(kw, code):
    assert fwd_s(**kw) == code
    assert binding.lib.gqa_last_error_string()


def test_fwd_strided_null_stride_arrays():
    assert binding.lib.gqa_attn_fwd_strided(P[0], P[1], P[2], P[3], 1, 4, 2, 8, 8, 32, None, None,
                                            0, 0, ctypes.c_float(0.1), BF16, None) == NULLP


def var(q=P[0], k=P[1], v=P[2], o=P[3], cq=P[4], ck=P[5], nseq=3, max_q=100, Hq=8, Hkv=2, d=64,
        causal=1, scale=0.125, dtype=BF16, stream=None):
    return binding.lib.gqa_attn_fwd_varlen(q, k, v, o, cq, ck, nseq, max_q, Hq, Hkv, d, causal,
                                           ctypes.c_float(scale), dtype, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(o=None), NULLP), (dict(cq=None), NULLP), (dict(ck=None), NULLP),
    (dict(nseq=0), SHAPE), (dict(max_q=0), SHAPE), (dict(max_q=(1 << 30) + 1), SHAPE),
    (dict(Hq=0), SHAPE), (dict(d=0), SHAPE),
    (dict(Hkv=2 ** 17, Hq=2 ** 17, d=128), SHAPE),       # 64 key rows past 2 GiB
    (dict(nseq=2 ** 20, max_q=2 ** 20, Hq=64, Hkv=64), SHAPE),  # too many work units
    (dict(Hq=6, Hkv=4), GROUP),
    (dict(d=48), UNSUP), (dict(dtype=2), UNSUP), (dict(scale=float("inf")), UNSUP),
    (dict(k=ctypes.c_void_p(0x20008)), UNSUP), (dict(cq=ctypes.c_void_p(0x50002)), UNSUP),
])
def test_fwd_varlen_rejects_invalid_arguments(kw, code):
    assert var(**kw) == code
    assert binding.lib.gqa_last_error_string()


def test_varlen_binding_checks_tensors_before_the_library():
    q = torch.zeros(10, 4, 32, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.attn_fwd_varlen(q, q[:, :2], q[:, :2], cu, cu, 6)  # CPU tensors are refused


def app(q=P[0], kn=P[6], vn=P[7], kc=P[1], vc=P[2], pos=P[4], o=P[3], B=8, Hq=12, Hkv=2,
        Smax=2048, d=128, scale=0.09, dtype=BF16, ws=P[5], ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = binding.decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    return binding.lib.gqa_attn_decode_append(q, kn, vn, kc, vc, pos, o, B, Hq, Hkv, Smax, d,
                                              ctypes.c_float(scale), dtype, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(kn=None), NULLP), (dict(vn=None), NULLP),
    (dict(kc=None), NULLP), (dict(vc=None), NULLP), (dict(pos=None), NULLP),
    (dict(o=None), NULLP),
    (dict(B=0), SHAPE), (dict(Smax=0), SHAPE), (dict(Hq=-2), SHAPE),
    (dict(Smax=2 ** 25, d=128), SHAPE),
    (dict(Hq=12, Hkv=5), GROUP),
    (dict(d=48), UNSUP), (dict(dtype=3), UNSUP), (dict(scale=float("nan")), UNSUP),
    (dict(kn=ctypes.c_void_p(0x30004)), UNSUP), (dict(vn=ctypes.c_void_p(0x30008)), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=64), WS),
])
def test_decode_append_rejects_invalid_arguments(kw, code):
    assert app(**kw) == code
    assert binding.lib.gqa_last_error_string()


def test_decode_workspace_bytes():
    ws = binding.decode_workspace_bytes
    # B * Hq * ceil(Smax / 32) partial records of d accumulators + max + sum,
    # padded to d + 4 fp32 so each record starts 16-byte aligned
    assert ws(8, 12, 2, 2048, 128) == 8 * 12 * 64 * 132 * 4
    assert ws(1, 1, 1, 1, 32) == 1 * 1 * 1 * 36 * 4
    assert ws(2, 4, 2, 33, 64) == 2 * 4 * 2 * 68 * 4
    for bad in [(0, 1, 1, 1, 32), (1, 3, 2, 1, 32), (1, 1, 1, 0, 32), (1, 1, 1, 8, 48)]:
        assert ws(*bad) == 0


def slt(q=P[0], kn=None, vn=None, kc=P[1], vc=P[2], ncache=16, slots=P[4], lens=P[5], o=P[3],
        B=8, Hq=12, Hkv=2, Smax=2048, d=128, scale=0.09, dtype=BF16, ws=P[6], ws_bytes=None,
        stream=None):
    if ws_bytes is None:
        ws_bytes = binding.decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    return binding.lib.gqa_attn_decode_slots(q, kn, vn, kc, vc, ncache, slots, lens, o, B, Hq,
                                             Hkv, Smax, d, ctypes.c_float(scale), dtype, ws,
                                             ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(kc=None), NULLP), (dict(slots=None), NULLP),
    (dict(lens=None), NULLP), (dict(o=None), NULLP), (dict(kn=P[7]), NULLP),
    (dict(vn=P[7]), NULLP),
    (dict(ncache=0), SHAPE), (dict(B=0), SHAPE), (dict(Smax=-1), SHAPE),
    (dict(Hq=12, Hkv=5), GROUP),
    (dict(d=48), UNSUP), (dict(dtype=7), UNSUP), (dict(scale=float("nan")), UNSUP),
    (dict(kn=ctypes.c_void_p(0x30004), vn=P[7]), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=64), WS),
])
def test_decode_slots_rejects_invalid_arguments(kw, code):
    assert slt(**kw) == code
    assert binding.lib.gqa_last_error_string()


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid arguments would launch on a GPU")
def test_valid_call_without_gpu_reports_no_device():
    assert fwd() == NODEV
    assert b"device" in binding.lib.gqa_last_error_string()
    assert dec() == NODEV
    assert dec_na() == NODEV
    assert app() == NODEV
    assert fwd_s() == NODEV
    assert var() == NODEV
    assert slt() == NODEV
    assert slt(kn=P[7], vn=P[0]) == NODEV
    # zero K/V batch stride (broadcast reads) is valid
    assert fwd_s(kvs=(0, 64, 128)) == NODEV


def test_binding_checks_tensors_before_the_library():
    q = torch.zeros(1, 4, 8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_fwd(q, q[:, :2], q[:, :2])  # CPU tensors are refused
    with pytest.raises(ValueError):
        binding.attn_fwd(q.float(), q[:, :2], q[:, :2])
    with pytest.raises(ValueError):
        binding.attn_decode(q[:, :, 0], q, q, torch.zeros(1, dtype=torch.int32))


# ---------------------------------------------------------------- backward
PB = [ctypes.c_void_p(0x10000 * (n + 1)) for n in range(9)]


def bwd(q=PB[0], k=PB[1], v=PB[2], o=PB[3], do=PB[4], dq=PB[5], dk=PB[6], dv=PB[7], B=1, Hq=4,
        Hkv=2, Nq=64, Nk=64, d=32, causal=0, q_offset=0, scale=0.17, dtype=BF16, ws=PB[8],
        ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = binding.bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    return binding.lib.gqa_attn_bwd(q, k, v, o, do, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal,
                                    q_offset, ctypes.c_float(scale), dtype, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(o=None), NULLP), (dict(do=None), NULLP), (dict(dq=None), NULLP),
    (dict(dk=None), NULLP), (dict(dv=None), NULLP),
    (dict(B=0), SHAPE), (dict(Nq=0), SHAPE), (dict(Nk=-3), SHAPE),
    (dict(causal=1, q_offset=-1), SHAPE), (dict(Nk=2 ** 30, d=32), SHAPE),
    (dict(Hq=6, Hkv=4), GROUP),
    (dict(dtype=7), UNSUP), (dict(d=48), UNSUP), (dict(scale=0.0), UNSUP),
    (dict(scale=-0.1), UNSUP), (dict(scale=float("inf")), UNSUP),
    (dict(dq=ctypes.c_void_p(0x10008)), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=64), WS), (dict(ws=ctypes.c_void_p(0x10004)), WS),
])
def test_bwd_rejects_invalid_arguments(kw, code):
    assert bwd(**kw) == code
    assert binding.lib.gqa_last_error_string()


def test_bwd_workspace_bytes():
    ws = binding.bwd_workspace_bytes
    # two fp32 row statistics (log-sum-exp and D) per query row, rounded up to
    # 16 bytes, then P query parts' fp32 dK and dV, P = min(16, ceil(1024 /
    # key blocks)) with ceil(Nk / 64) key blocks per (batch, K/V head), none
    # when P = 1
    assert ws(1, 32, 8, 2048, 2048, 128) == 2 * 32 * 2048 * 4 + 4 * 2 * 8 * 2048 * 128 * 4
    assert ws(1, 16, 16, 2048, 2048, 64) == 2 * 16 * 2048 * 4 + 2 * 2 * 16 * 2048 * 64 * 4
    assert ws(1, 32, 1, 4096, 4096, 128) == 2 * 32 * 4096 * 4 + 16 * 2 * 4096 * 128 * 4
    assert ws(3, 5, 5, 7, 9, 32) == 848 + 16 * 2 * 3 * 5 * 9 * 32 * 4  # 840 bytes -> 848
    assert ws(8, 8, 8, 2048, 2048, 128) == 2 * 8 * 8 * 2048 * 4  # 2048 key blocks: one part
    for bad in [(0, 1, 1, 1, 1, 32), (1, 3, 2, 1, 1, 32), (1, 1, 1, 0, 1, 32),
                (1, 1, 1, 1, 0, 32), (1, 1, 1, 1, 1, 48)]:
        assert ws(*bad) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid arguments would launch on a GPU")
def test_valid_bwd_call_without_gpu_reports_no_device():
    assert bwd() == NODEV
    assert bwd(causal=1, q_offset=5, dtype=F32, d=128) == NODEV


# ---------------------------------------------------------------- mixed batch
PM = [ctypes.c_void_p(0x10000 * (n + 1)) for n in range(11)]
NUL = ctypes.c_void_p(0)


def mixed(q=PM[0], k=PM[1], v=PM[2], o=PM[3], B=1, Nq=64, Nk=128, q_offset=64, qd=PM[4],
          kc=PM[5], vc=PM[6], lens=PM[7], od=PM[8], Bd=2, Smax=256, Hq=4, Hkv=2, d=64,
          scale=0.125, dtype=BF16, ws=PM[9], ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = binding.lib.gqa_attn_decode_workspace_bytes(max(Bd, 1), Hq, Hkv, max(Smax, 1),
                                                               d)
    return binding.lib.gqa_attn_mixed(q, k, v, o, B, Nq, Nk, q_offset, qd, kc, vc, lens, od, Bd,
                                      Smax, Hq, Hkv, d, scale, dtype, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), SHAPE), (dict(Bd=-1), SHAPE),
    (dict(q=NUL), NULLP), (dict(o=NUL), NULLP), (dict(qd=NUL), NULLP),
    (dict(lens=NUL), NULLP), (dict(od=NUL), NULLP),
    (dict(Nq=0), SHAPE), (dict(q_offset=-1), SHAPE), (dict(Smax=0), SHAPE),
    (dict(Hq=6, Hkv=4), GROUP), (dict(d=96), UNSUP), (dict(dtype=5), UNSUP),
    (dict(scale=float("nan")), UNSUP), (dict(ws=NUL), WS), (dict(ws_bytes=16), WS),
    (dict(kc=ctypes.c_void_p(0x10008)), UNSUP), (dict(q=ctypes.c_void_p(0x10004)), UNSUP),
    (dict(Bd=70000, ws_bytes=1 << 40), SHAPE),
    (dict(Nq=1 << 28, d=128), SHAPE), (dict(Hq=1 << 30, Hkv=1 << 30, Nq=1 << 24), SHAPE),
], ids=lambda x: str(x))
def test_mixed_rejects_invalid_arguments(kw, code):
    assert mixed(**kw) == code
    assert binding.lib.gqa_last_error_string() != b""


def test_mixed_absent_parts_need_no_pointers():
    # both parts empty: nothing to do, and no pointer is looked at
    assert mixed(q=NUL, k=NUL, v=NUL, o=NUL, B=0, qd=NUL, kc=NUL, vc=NUL, lens=NUL, od=NUL, Bd=0,
                 ws=NUL, ws_bytes=0) == OK
    # an absent part's sizes and pointers are not checked
    assert mixed(q=NUL, B=0, Nq=0, Nk=0, q_offset=-5, qd=NUL, Bd=0, Smax=0, ws=NUL,
                 ws_bytes=0) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid arguments would launch on a GPU")
def test_valid_mixed_call_without_gpu_reports_no_device():
    assert mixed() == NODEV
    assert mixed(q=NUL, k=NUL, v=NUL, o=NUL, B=0) == NODEV           # decode rows only
    assert mixed(qd=NUL, kc=NUL, vc=NUL, lens=NUL, od=NUL, Bd=0, ws=NUL, ws_bytes=0) == NODEV


def test_mixed_binding_checks_parts_before_the_library():
    q = torch.zeros(1, 4, 8, 32, dtype=torch.bfloat16)
    assert binding.attn_mixed(None, None, None, 0, None, None, None, None) == (None, None)
    with pytest.raises(ValueError):
        binding.attn_mixed(q, None, None, 0, None, None, None, None)
    with pytest.raises(ValueError):
        binding.attn_mixed(None, None, None, 0, q[:, :, 0], q, None, None)
    with pytest.raises(ValueError):  # CPU tensors are refused
        binding.attn_mixed(q, q[:, :2], q[:, :2], 0, None, None, None, None)


def test_microbench_library_exports_and_rejects_bad_arguments():
    """The measurement library (bench.py's machine peaks and --lds-probe) loads,
    exports its entry points, and refuses invalid arguments before any
    HIP call (return 1)."""
    path = os.path.join(os.path.dirname(binding.LIBRARY), "libgqa_microbench.so")
    lib = ctypes.CDLL(path)
    for name in ("gqa_mb_mfma_bf16", "gqa_mb_read", "gqa_mb_lds", "gqa_mb_valu"):
        assert hasattr(lib, name), name
    lib.gqa_mb_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p]
    sink = ctypes.c_void_p(16)  # never dereferenced: every call below is refused first
    assert lib.gqa_mb_lds(-1, 1, 1, sink, None) == 1
    assert lib.gqa_mb_lds(11, 1, 1, sink, None) == 1
    assert lib.gqa_mb_lds(0, 0, 1, sink, None) == 1
    assert lib.gqa_mb_lds(0, 1, 0, sink, None) == 1
    assert lib.gqa_mb_lds(0, 1, 1, None, None) == 1
    lib.gqa_mb_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gqa_mb_valu(2, 1, 1, sink, sink, None) == 1
    assert lib.gqa_mb_valu(0, 1, 1, None, sink, None) == 1
