"""ctypes binding of libgqa_attn.so (C ABI in include/gqa_attn.h).

Argument marshalling only: shape/dtype/device checks on torch tensors, output
and workspace allocation through torch's caching allocator, and the current
torch stream handed to the library.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.  If the library is
missing, loading it raises ``ImportError`` -- it has to be built first
(``python -m mqa_flashattention_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgqa_attn.so")

GQA_DTYPE_F32 = 0
GQA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: GQA_DTYPE_F32, torch.bfloat16: GQA_DTYPE_BF16}

STATUS_NAMES = {
    0: "GQA_OK", 1: "GQA_ERR_NULL_POINTER", 2: "GQA_ERR_BAD_SHAPE", 3: "GQA_ERR_HEAD_GROUPING",
    4: "GQA_ERR_UNSUPPORTED", 5: "GQA_ERR_WORKSPACE", 6: "GQA_ERR_NO_DEVICE", 7: "GQA_ERR_HIP",
}
EXPORTED = ("gqa_attn_fwd", "gqa_attn_fwd_strided", "gqa_attn_fwd_varlen", "gqa_attn_decode",
            "gqa_attn_decode_noalloc", "gqa_attn_decode_append", "gqa_attn_decode_slots",
            "gqa_attn_decode_workspace_bytes", "gqa_attn_bwd", "gqa_attn_bwd_workspace_bytes",
            "gqa_attn_mixed", "gqa_status_string", "gqa_last_error_string")


class GqaError(RuntimeError):
    """A non-zero status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is not built; run `python -m mqa_flashattention_amd.build`")
    lib = ctypes.CDLL(LIBRARY)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.gqa_attn_fwd.restype = i
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.gqa_attn_fwd_strided.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i, i, f,
                                         i, vp]
    lib.gqa_attn_fwd_strided.restype = i
    lib.gqa_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.gqa_attn_fwd_varlen.restype = i
    lib.gqa_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gqa_attn_decode_workspace_bytes.restype = sz
    lib.gqa_attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.gqa_attn_decode.restype = i
    lib.gqa_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.gqa_attn_decode_noalloc.restype = i
    lib.gqa_attn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp,
                                           sz, vp]
    lib.gqa_attn_decode_append.restype = i
    lib.gqa_attn_decode_slots.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, f, i,
                                          vp, sz, vp]
    lib.gqa_attn_decode_slots.restype = i
    lib.gqa_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gqa_attn_bwd_workspace_bytes.restype = sz
    lib.gqa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp,
                                 sz, vp]
    lib.gqa_attn_bwd.restype = i
    lib.gqa_attn_mixed.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, vp, i, i, i, i, i,
                                   f, i, vp, sz, vp]
    lib.gqa_attn_mixed.restype = i
    lib.gqa_status_string.argtypes = [i]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_last_error_string.argtypes = []
    lib.gqa_last_error_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def library_path() -> str:
    return LIBRARY


def _raise(status: int) -> None:
    if status != 0:
        detail = lib.gqa_last_error_string().decode(errors="replace")
        raise GqaError(status, detail or lib.gqa_status_string(status).decode())


def _check_tensor(name: str, t: torch.Tensor, ndim: int, dtype: torch.dtype, device,
                  contiguous: bool = True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (a GPU device), got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last (head) dimension must be contiguous")


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             q_offset: int = 0, scale: float | None = None,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """O = softmax(scale * Q K^T [causal at q_offset]) V via gqa_attn_fwd.

    q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d], all bfloat16 or all float32,
    contiguous, on one GPU.  Query head h reads K/V head h // (Hq // Hkv).
    scale defaults to 1/sqrt(d)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 4, q.dtype, dev)
    _check_tensor("k", k, 4, q.dtype, dev)
    _check_tensor("v", v, 4, q.dtype, dev)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 4, q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), int(q_offset),
                              float(scale), _DTYPES[q.dtype], _stream_handle(dev))
    _raise(st)
    return out


def attn_fwd_strided(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                     q_offset: int = 0, scale: float | None = None,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """attn_fwd over strided views, via gqa_attn_fwd_strided.

    q [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d] are indexed as logical
    (batch, head, token, d) views with any strides whose last one is 1, e.g.
    ``x.transpose(1, 2)`` of a token-major [B, N, H, d] tensor: no copy is
    made.  k and v must share their strides; out must have the strides of q
    (it is allocated with them when not given)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 4, q.dtype, dev, contiguous=False)
    _check_tensor("k", k, 4, q.dtype, dev, contiguous=False)
    _check_tensor("v", v, 4, q.dtype, dev, contiguous=False)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if k.stride() != v.stride():
        raise ValueError(f"k and v must share strides, got {k.stride()} and {v.stride()}")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    else:
        _check_tensor("out", out, 4, q.dtype, dev, contiguous=False)
        if tuple(out.shape) != tuple(q.shape) or out.stride() != q.stride():
            raise ValueError("out must have the shape and strides of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qs = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    kvs = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    with torch.cuda.device(dev):
        st = lib.gqa_attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      B, Hq, Hkv, Nq, Nk, d, qs, kvs, int(bool(causal)),
                                      int(q_offset), float(scale), _DTYPES[q.dtype],
                                      _stream_handle(dev))
    _raise(st)
    return out


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int, *,
                    causal: bool = False, scale: float | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed variable-length forward via gqa_attn_fwd_varlen.

    q [total_q, Hq, d], k and v [total_k, Hkv, d] (token-major, contiguous,
    one dtype, one GPU); cu_seqlens_q / cu_seqlens_k int32 [nseq + 1] on the
    same GPU (sequence s owns rows [cu[s], cu[s+1])); max_seqlen_q: a host
    int >= every sequence's query count.  Each sequence's queries are its
    last tokens; causal: query i sees keys j <= Nk - Nq + i.  scale defaults
    to 1/sqrt(d)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 3, q.dtype, dev)
    _check_tensor("k", k, 3, q.dtype, dev)
    _check_tensor("v", v, 3, q.dtype, dev)
    _check_tensor("cu_seqlens_q", cu_seqlens_q, 1, torch.int32, dev)
    _check_tensor("cu_seqlens_k", cu_seqlens_k, 1, torch.int32, dev)
    _, Hq, d = q.shape
    _, Hkv, _ = k.shape
    if k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    nseq = cu_seqlens_q.shape[0] - 1
    if nseq < 1 or cu_seqlens_k.shape[0] != nseq + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold nseq + 1 >= 2 offsets")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 3, q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), nseq,
                                     int(max_seqlen_q), Hq, Hkv, d, int(bool(causal)),
                                     float(scale), _DTYPES[q.dtype], _stream_handle(dev))
    _raise(st)
    return out


def bwd_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(lib.gqa_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             dout: torch.Tensor, *, causal: bool = False, q_offset: int = 0,
             scale: float | None = None, workspace: torch.Tensor | None = None):
    """(dq, dk, dv) of a loss with dL/do = dout, via gqa_attn_bwd.

    q, o, dout [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d]; all of one dtype,
    contiguous, on one GPU; o is the output of attn_fwd on the same inputs and
    options.  dk, dv are summed over the query heads of each K/V head.
    scale defaults to 1/sqrt(d) and must be > 0."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, 4, q.dtype, dev)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have the shape of q")
    need = bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), int(q_offset),
                              float(scale), _DTYPES[q.dtype], workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream_handle(dev))
    _raise(st)
    return dq, dk, dv


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Smax: int, d: int) -> int:
    return int(lib.gqa_attn_decode_workspace_bytes(B, Hq, Hkv, Smax, d))


def attn_decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                seqlens: torch.Tensor, *, scale: float | None = None,
                out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Single-token decode via gqa_attn_decode.

    q [B, Hq, d]; kcache, vcache [B, Hkv, Smax, d]; seqlens int32 [B] on the
    same GPU.  Row b attends slots [0, clamp(seqlens[b], 0, Smax)).  The
    workspace (uint8, at least decode_workspace_bytes(...)) is allocated when
    not given."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 3, q.dtype, dev)
    _check_tensor("kcache", kcache, 4, q.dtype, dev)
    _check_tensor("vcache", vcache, 4, q.dtype, dev)
    _check_tensor("seqlens", seqlens, 1, torch.int32, dev)
    B, Hq, d = q.shape
    _, Hkv, Smax, _ = kcache.shape
    if kcache.shape[0] != B or kcache.shape[3] != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} kcache{tuple(kcache.shape)}")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must have B entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 3, q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    need = decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                                 seqlens.data_ptr(), out.data_ptr(), B, Hq, Hkv, Smax, d,
                                 float(scale), _DTYPES[q.dtype], workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_handle(dev))
    _raise(st)
    return out


# Bytes of the static scratch behind gqa_attn_decode_noalloc (the header's
# GQA_DECODE_NOALLOC_SCRATCH_BYTES).
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def attn_decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                        seqlens: torch.Tensor, out: torch.Tensor, *,
                        scale: float | None = None) -> torch.Tensor:
    """attn_decode via gqa_attn_decode_noalloc: no workspace, and nothing is
    allocated -- out must be given (shape and dtype of q); the split records
    live in the library's static scratch on the GPU.  Calls that may overlap
    on one GPU must not use it."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 3, q.dtype, dev)
    _check_tensor("kcache", kcache, 4, q.dtype, dev)
    _check_tensor("vcache", vcache, 4, q.dtype, dev)
    _check_tensor("seqlens", seqlens, 1, torch.int32, dev)
    _check_tensor("out", out, 3, q.dtype, dev)
    B, Hq, d = q.shape
    _, Hkv, Smax, _ = kcache.shape
    if kcache.shape[0] != B or kcache.shape[3] != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} kcache{tuple(kcache.shape)}")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must have B entries")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_decode_noalloc(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                                         seqlens.data_ptr(), out.data_ptr(), B, Hq, Hkv, Smax,
                                         d, float(scale), _DTYPES[q.dtype], _stream_handle(dev))
    _raise(st)
    return out


def attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       kcache: torch.Tensor, vcache: torch.Tensor, positions: torch.Tensor, *,
                       scale: float | None = None, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode step with append via gqa_attn_decode_append.

    q [B, Hq, d]; k_new, v_new [B, Hkv, d]; kcache, vcache [B, Hkv, Smax, d]
    (written in place); positions int32 [B] on the same GPU.  Row b with
    p = positions[b] in [0, Smax) stores its new K/V rows in slot p and
    attends slots [0, p]; other rows are inactive (zero output, no store).
    The positions are not advanced."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 3, q.dtype, dev)
    _check_tensor("k_new", k_new, 3, q.dtype, dev)
    _check_tensor("v_new", v_new, 3, q.dtype, dev)
    _check_tensor("kcache", kcache, 4, q.dtype, dev)
    _check_tensor("vcache", vcache, 4, q.dtype, dev)
    _check_tensor("positions", positions, 1, torch.int32, dev)
    B, Hq, d = q.shape
    _, Hkv, Smax, _ = kcache.shape
    if kcache.shape[0] != B or kcache.shape[3] != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} kcache{tuple(kcache.shape)}")
    if tuple(k_new.shape) != (B, Hkv, d) or tuple(v_new.shape) != (B, Hkv, d):
        raise ValueError(f"k_new and v_new must be [B, Hkv, d] = {(B, Hkv, d)}")
    if positions.shape[0] != B:
        raise ValueError("positions must have B entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 3, q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    need = decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                        kcache.data_ptr(), vcache.data_ptr(),
                                        positions.data_ptr(), out.data_ptr(), B, Hq, Hkv, Smax,
                                        d, float(scale), _DTYPES[q.dtype],
                                        workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_handle(dev))
    _raise(st)
    return out


def attn_decode_slots(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                      slots: torch.Tensor, lengths: torch.Tensor, *,
                      k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None,
                      scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode over a cache pool through a slot table, via gqa_attn_decode_slots.

    q [B, Hq, d]; kcache, vcache [Ncache, Hkv, Smax, d]; slots and lengths
    int32 [B] on the same GPU.  Row b reads cache row slots[b] (a slot outside
    [0, Ncache) makes the row inactive: zero output, no cache access).
    Without k_new / v_new, lengths[b] is the row's cached length; with them
    ([B, Hkv, d] each) it is the new token's position p, whose K/V rows are
    written to cache row slots[b] at p (in place) before the row attends
    positions 0 .. p."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _check_tensor("q", q, 3, q.dtype, dev)
    _check_tensor("kcache", kcache, 4, q.dtype, dev)
    _check_tensor("vcache", vcache, 4, q.dtype, dev)
    _check_tensor("slots", slots, 1, torch.int32, dev)
    _check_tensor("lengths", lengths, 1, torch.int32, dev)
    B, Hq, d = q.shape
    Ncache, Hkv, Smax, _ = kcache.shape
    if kcache.shape[3] != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} kcache{tuple(kcache.shape)}")
    if slots.shape[0] != B or lengths.shape[0] != B:
        raise ValueError("slots and lengths must have B entries")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _check_tensor("k_new", k_new, 3, q.dtype, dev)
        _check_tensor("v_new", v_new, 3, q.dtype, dev)
        if tuple(k_new.shape) != (B, Hkv, d) or tuple(v_new.shape) != (B, Hkv, d):
            raise ValueError(f"k_new and v_new must be [B, Hkv, d] = {(B, Hkv, d)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 3, q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    need = decode_workspace_bytes(B, Hq, Hkv, Smax, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_decode_slots(q.data_ptr(),
                                       k_new.data_ptr() if k_new is not None else None,
                                       v_new.data_ptr() if v_new is not None else None,
                                       kcache.data_ptr(), vcache.data_ptr(), Ncache,
                                       slots.data_ptr(), lengths.data_ptr(), out.data_ptr(), B,
                                       Hq, Hkv, Smax, d, float(scale), _DTYPES[q.dtype],
                                       workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(),
                                       _stream_handle(dev))
    _raise(st)
    return out


def attn_mixed(q: torch.Tensor | None, k: torch.Tensor | None, v: torch.Tensor | None,
               q_offset: int, qd: torch.Tensor | None, kcache: torch.Tensor | None,
               vcache: torch.Tensor | None, seqlens: torch.Tensor | None, *,
               scale: float | None = None, out: torch.Tensor | None = None,
               out_decode: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None):
    """A chunked-prefill chunk and decode rows in one launch via gqa_attn_mixed.

    Chunk: q [B, Hq, Nq, d], k, v [B, Hkv, Nk, d], causal, query row i at
    position q_offset + i (q is None: no chunk).  Decode rows: qd [Bd, Hq, d],
    kcache, vcache [Bd, Hkv, Smax, d], seqlens int32 [Bd] (qd is None: no
    decode rows).  Returns (o, od); the missing part's entry is None."""
    if q is not None and (k is None or v is None):
        raise ValueError("a chunk needs q, k and v")
    if qd is not None and (kcache is None or vcache is None or seqlens is None):
        raise ValueError("decode rows need qd, kcache, vcache and seqlens")
    ref = q if q is not None else qd
    if ref is None:
        return None, None
    if ref.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {ref.dtype}")
    dev = ref.device
    B = Nq = Nk = 0
    Bd = Smax = 0
    Hq, d = ref.shape[1], ref.shape[-1]
    Hkv = (k if q is not None else kcache).shape[1]
    nul = ctypes.c_void_p(0)
    ptrs = [nul] * 4
    if q is not None:
        _check_tensor("q", q, 4, ref.dtype, dev)
        _check_tensor("k", k, 4, ref.dtype, dev)
        _check_tensor("v", v, 4, ref.dtype, dev)
        B, _, Nq, _ = q.shape
        Nk = k.shape[2]
        if (tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape)
                or q.shape[1] != Hq or q.shape[3] != d):
            raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor("out", out, 4, ref.dtype, dev)
            if tuple(out.shape) != tuple(q.shape):
                raise ValueError("out must have the shape of q")
        ptrs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()]
    else:
        out = None
    dptrs = [nul] * 5
    ws_ptr, ws_bytes = nul, 0
    if qd is not None:
        _check_tensor("qd", qd, 3, ref.dtype, dev)
        _check_tensor("kcache", kcache, 4, ref.dtype, dev)
        _check_tensor("vcache", vcache, 4, ref.dtype, dev)
        _check_tensor("seqlens", seqlens, 1, torch.int32, dev)
        Bd = qd.shape[0]
        Smax = kcache.shape[2]
        if (tuple(qd.shape) != (Bd, Hq, d) or tuple(kcache.shape) != (Bd, Hkv, Smax, d)
                or tuple(vcache.shape) != tuple(kcache.shape) or seqlens.shape[0] != Bd):
            raise ValueError(f"shape mismatch qd{tuple(qd.shape)} kcache{tuple(kcache.shape)}")
        if out_decode is None:
            out_decode = torch.empty_like(qd)
        else:
            _check_tensor("out_decode", out_decode, 3, ref.dtype, dev)
            if tuple(out_decode.shape) != tuple(qd.shape):
                raise ValueError("out_decode must have the shape of qd")
        need = decode_workspace_bytes(Bd, Hq, Hkv, Smax, d)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        elif workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the GPU of the inputs")
        dptrs = [qd.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), seqlens.data_ptr(),
                 out_decode.data_ptr()]
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        out_decode = None
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(dev):
        st = lib.gqa_attn_mixed(*ptrs, B, Nq, Nk, int(q_offset), *dptrs, Bd, Smax, Hq, Hkv, d,
                                float(scale), _DTYPES[ref.dtype], ws_ptr, ws_bytes,
                                _stream_handle(dev))
    _raise(st)
    return out, out_decode
