"""GPU test of gqa_attn_decode_noalloc, the decode entry point that allocates
nothing (its split records live in a static device array).

Called through the C ABI and compared with gqa_attn_decode on the same
inputs: bit for bit (same kernels, same splits), and against the CPU fp64
oracle within the bf16 tolerance.  Two calls in a row, the second with a
smaller input, so stale records of the first cannot leak into the second.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from mqa_flashattention_amd import binding
from mqa_flashattention_amd.workloads import WORKLOADS, DecodeShape, decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc_via_abi(q, kc, vc, lens, out, scale):
    """One gqa_attn_decode_noalloc call with raw pointers."""
    B, Hq, d = q.shape
    _, Hkv, Smax, _ = kc.shape
    st = binding.lib.gqa_attn_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
        ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(lens.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), B, Hq, Hkv, Smax, d, ctypes.c_float(scale),
        binding.GQA_DTYPE_BF16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, binding.lib.gqa_last_error_string().decode()


def test_noalloc_decode_matches_workspace_decode_twice():
    shapes = [WORKLOADS["kv_decode_b8"].decode,          # the batch-8 decode workload
              DecodeShape(3, 12, 2, 700, 128, 1, 700)]   # then a smaller one
    for n, s in enumerate(shapes):
        q_h, kc_h, vc_h, lens_h = decode_inputs(s, 40 + n)
        q, kc, vc, lens = (t.to(DEV) for t in (q_h, kc_h, vc_h, lens_h))
        assert binding.decode_workspace_bytes(s.B, s.Hq, s.Hkv, s.Smax, s.d) <= \
            binding.DECODE_NOALLOC_SCRATCH_BYTES
        want = binding.attn_decode(q, kc, vc, lens, scale=s.scale)
        out = torch.full_like(q, float("nan"))
        _noalloc_via_abi(q, kc, vc, lens, out, s.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {n}: differs from gqa_attn_decode"
        ref = oracle.attn_decode(q_h, kc_h, vc_h, lens_h, scale=s.scale)
        err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
        assert err <= 2e-2, f"call {n}: max abs error {err}"


def test_noalloc_decode_rejects_oversized_calls():
    """A decode whose split records exceed the static scratch is refused with
    GQA_ERR_WORKSPACE before anything is launched."""
    B, Hq, Hkv, Smax, d = 64, 32, 8, 32768, 128
    assert binding.decode_workspace_bytes(B, Hq, Hkv, Smax, d) > \
        binding.DECODE_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x10000)
    st = binding.lib.gqa_attn_decode_noalloc(p, p, p, p, p, B, Hq, Hkv, Smax, d,
                                             ctypes.c_float(0.1), binding.GQA_DTYPE_BF16, None)
    assert st == 5
