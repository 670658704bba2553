"""CPU fp64 oracle for grouped-query attention forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product package: the two sides share nothing but the seeded
inputs handed to both.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, OpenMP over output
rows).  This module only compiles it with gcc and marshals numpy arrays.
Every function widens its inputs to float64 exactly before the call (bf16 and
fp32 values are exactly representable in fp64).

What it computes, with its sources, is written at the top of ``attn_oracle.c``:
the definition O = softmax(scale * Q K^T [causal, q_offset]) V with query head
h reading K/V head h // (Hq // Hkv) (BootstrapAI evolution log, "Kernel 9 --
GQA Flash Attention"), evaluated as max / exp-sum / weighted sum per row.  The decode step with
append first writes each active row's new K/V rows at its position (the
single-launch K/V store and per-row position table of the microLLM-rocm
optimization log, experiments 025, 083/084 and 098) and then attends slots
[0, position].  A mixed batch (a chunked-prefill chunk beside decode rows,
kaispace.site note "Chunked Prefill") is the two definitions side by side,
and a packed batch of sequences of different lengths (attn_fwd_varlen) is
the forward definition applied to each sequence on its own.
The backward gives dQ, dK, dV of a loss with dL/dO given,
the K/V gradients reduced over each K/V head's query heads (microLLM-rocm
optimization log, experiments 044 and 051-054).

Parity status: pinned (see tests/test_oracle.py -- library attention routine
on random shapes, closed forms, invariants, and planted-mistake checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "libattn_oracle.so")

_lock = threading.Lock()
_libs: dict[str, ctypes.CDLL] = {}

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.c_long


def compile_oracle(source: str = SOURCE, output: str = LIBRARY, strict: bool = True) -> str:
    """Compile the oracle C source into a shared library with gcc (-O2, IEEE).

    ``strict`` turns warnings into errors (the real source must build clean)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]
    if strict:
        cmd.append("-Werror")
    cmd += [source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def load(path: str = LIBRARY, build_if_missing: bool = True) -> ctypes.CDLL:
    """Load (compiling first if absent) an oracle library and declare its ABI."""
    with _lock:
        if path in _libs:
            return _libs[path]
        if not os.path.exists(path):
            if not build_if_missing:
                raise FileNotFoundError(path)
            compile_oracle(SOURCE, path)
        lib = ctypes.CDLL(path)
        lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, _dp, _lp, _lp, _lp, _lp, _lp, _lp,
                                        ctypes.c_int, _lp, ctypes.c_double]
        lib.oracle_attn_fwd_rows.argtypes = [_dp, _dp, _dp, _lp, _lp, _lp, _lp, _lp, _lp,
                                             ctypes.c_int, _lp, ctypes.c_double,
                                             ctypes.POINTER(ctypes.c_int64), _lp, _dp]
        lib.oracle_attn_probs.argtypes = [_dp, _dp, _dp, _lp, _lp, _lp, _lp, _lp, _lp,
                                          ctypes.c_int, _lp, ctypes.c_double,
                                          _lp, _lp, _lp, _dp]
        lib.oracle_attn_decode.argtypes = [_dp, _dp, _dp, ctypes.POINTER(ctypes.c_int32),
                                           _dp, _lp, _lp, _lp, _lp, _lp, ctypes.c_double]
        lib.oracle_attn_decode_append.argtypes = [_dp, _dp, _dp, _dp, _dp,
                                                  ctypes.POINTER(ctypes.c_int32), _dp,
                                                  _lp, _lp, _lp, _lp, _lp, ctypes.c_double]
        lib.oracle_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _lp, _lp, _lp, _lp,
                                        _lp, _lp, ctypes.c_int, _lp, ctypes.c_double]
        for name in ("oracle_attn_fwd", "oracle_attn_fwd_rows", "oracle_attn_probs",
                     "oracle_attn_decode", "oracle_attn_decode_append", "oracle_attn_bwd",
                     "oracle_num_threads"):
            getattr(lib, name).restype = ctypes.c_int
        _libs[path] = lib
        return lib


def _f64(x) -> np.ndarray:
    """Exact widening of a numpy array or (CPU) torch tensor to contiguous float64."""
    if hasattr(x, "detach"):  # torch tensor: widen in torch (bf16 has no numpy dtype)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def attn_fwd(q, k, v, *, causal: bool = False, q_offset: int = 0, scale: float | None = None,
             lib: ctypes.CDLL | None = None) -> np.ndarray:
    """O[B,Hq,Nq,d] (float64) for q[B,Hq,Nq,d], k,v[B,Hkv,Nk,d]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    _check(lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Nq, Nk, d,
                               int(bool(causal)), int(q_offset), float(scale)), "attn_fwd")
    return o


def attn_fwd_rows(q, k, v, row_ids, *, causal: bool = False, q_offset: int = 0,
                  scale: float | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Rows (b*Hq + h)*Nq + i of the forward output, as float64 [len(row_ids), d]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64))
    out = np.empty((ids.size, d), dtype=np.float64)
    _check(lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Nq, Nk, d,
                                    int(bool(causal)), int(q_offset), float(scale),
                                    ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    ids.size, _ptr(out)), "attn_fwd_rows")
    return out


def _varlen_offsets(cu) -> np.ndarray:
    if hasattr(cu, "detach"):
        cu = cu.detach().to("cpu").numpy()
    return np.asarray(cu, dtype=np.int64)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool = False,
                    scale: float | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """O[total_q, Hq, d] (float64) for packed token-major q[total_q, Hq, d] and
    k, v[total_k, Hkv, d] holding several sequences back to back.

    Sequence s owns query rows [cu_q[s], cu_q[s+1]) and key rows
    [cu_k[s], cu_k[s+1]) (nseq + 1 offsets each, first 0).  Its output is the
    forward definition on its own tensors: query row i (0-based within the
    sequence) sits at position Nk_s - Nq_s + i -- the queries are the
    sequence's last Nq_s tokens, as a chunk of a prompt is (kaispace.site
    note "Chunked Prefill"), and the whole prompt when Nq_s = Nk_s -- and,
    causal, sees the keys j <= Nk_s - Nq_s + i.  A row that sees no key
    (Nk_s = 0, or causal rows i < Nq_s - Nk_s) is zero, as an empty decode
    row is.  Composed per sequence from attn_fwd; no arithmetic of its own."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq, ck = _varlen_offsets(cu_seqlens_q), _varlen_offsets(cu_seqlens_k)
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or cq.shape != ck.shape:
        raise ValueError("attn_fwd_varlen: q [Tq,Hq,d], k/v [Tk,Hkv,d], offsets [nseq+1]")
    d = q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
        nq, nk = q1 - q0, k1 - k0
        if nq <= 0 or nk <= 0:
            continue
        qs = q[q0:q1].transpose(1, 0, 2)[None]          # [1, Hq, Nq, d]
        ks = k[k0:k1].transpose(1, 0, 2)[None]          # [1, Hkv, Nk, d]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        if not causal:
            os_ = attn_fwd(qs, ks, vs, causal=False, scale=scale, lib=lib)
            o[q0:q1] = os_[0].transpose(1, 0, 2)
            continue
        off = nk - nq
        first = max(0, -off)                          # rows before it see no key
        if first >= nq:
            continue
        os_ = attn_fwd(qs[:, :, first:], ks, vs, causal=True, q_offset=off + first, scale=scale,
                       lib=lib)
        o[q0 + first:q1] = os_[0].transpose(1, 0, 2)
    return o


def attn_probs(q, k, v, b: int, h: int, i: int, *, causal: bool = False, q_offset: int = 0,
               scale: float | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Softmax weights [Nk] of query row (b, h, i); zero for masked keys."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    p = np.empty(Nk, dtype=np.float64)
    _check(lib.oracle_attn_probs(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Nq, Nk, d,
                                 int(bool(causal)), int(q_offset), float(scale), b, h, i,
                                 _ptr(p)), "attn_probs")
    return p


def attn_decode(q, kcache, vcache, seqlens, *, scale: float | None = None,
                lib: ctypes.CDLL | None = None) -> np.ndarray:
    """O[B,Hq,d] for q[B,Hq,d], caches [B,Hkv,Smax,d], seqlens int[B]."""
    lib = lib or load()
    q, kc, vc = _f64(q), _f64(kcache), _f64(vcache)
    if hasattr(seqlens, "detach"):
        seqlens = seqlens.detach().to("cpu").numpy()
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, Hq, d = q.shape
    Hkv, Smax = kc.shape[1], kc.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    _check(lib.oracle_attn_decode(_ptr(q), _ptr(kc), _ptr(vc),
                                  sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(o),
                                  B, Hq, Hkv, Smax, d, float(scale)), "attn_decode")
    return o


def attn_decode_append(q, k_new, v_new, kcache, vcache, positions, *,
                       scale: float | None = None, lib: ctypes.CDLL | None = None):
    """Decode step with append: returns (O[B,Hq,d], K cache, V cache) as float64.

    q[B,Hq,d], k_new/v_new[B,Hkv,d], caches [B,Hkv,Smax,d], positions int[B].
    Row b with 0 <= positions[b] < Smax writes its new K/V rows into slot
    positions[b] and attends slots [0, positions[b]]; other rows are inactive
    (no write, zero output).  The input caches are not modified: the updated
    caches are returned as new arrays."""
    lib = lib or load()
    q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
    kc, vc = _f64(kcache).copy(), _f64(vcache).copy()
    if hasattr(positions, "detach"):
        positions = positions.detach().to("cpu").numpy()
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    B, Hq, d = q.shape
    Hkv, Smax = kc.shape[1], kc.shape[2]
    if kn.shape != (B, Hkv, d) or vn.shape != (B, Hkv, d) or pos.shape != (B,):
        raise ValueError("attn_decode_append: k_new/v_new must be [B,Hkv,d], positions [B]")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    _check(lib.oracle_attn_decode_append(_ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc),
                                         pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         _ptr(o), B, Hq, Hkv, Smax, d, float(scale)),
           "attn_decode_append")
    return o, kc, vc


def attn_decode_slots(q, kcache, vcache, slots, lengths, *, k_new=None, v_new=None,
                      scale: float | None = None, lib: ctypes.CDLL | None = None):
    """Decode over a pool of cache rows through a slot table (float64).

    Row b of the batch uses cache row slots[b] of kcache, vcache
    [Ncache, Hkv, Smax, d] -- positions reached through a small per-row
    table (microLLM-rocm optimization log, experiment 098); a slot outside
    [0, Ncache) makes the row inactive (zero output, no cache access), which
    leaves it out of the batch's work as active-row compaction does
    (experiment 097).  Without k_new / v_new: the decode definition over the
    row's cache row with lengths[b] cached tokens; returns O.  With them:
    the decode step with append on that cache row at position lengths[b];
    returns (O, K pool, V pool) with the pools updated (inputs untouched).
    Composed from attn_decode / attn_decode_append on the gathered rows --
    no arithmetic of its own."""
    kc, vc = _f64(kcache), _f64(vcache)
    if hasattr(slots, "detach"):
        slots = slots.detach().to("cpu").numpy()
    if hasattr(lengths, "detach"):
        lengths = lengths.detach().to("cpu").numpy()
    sl = np.asarray(slots, dtype=np.int64)
    ln = np.asarray(lengths, dtype=np.int64)
    ncache = kc.shape[0]
    active = (sl >= 0) & (sl < ncache)
    rows = np.where(active, sl, 0)
    kg, vg = kc[rows], vc[rows]                       # [B, Hkv, Smax, d]
    if k_new is None:
        eff = np.where(active, ln, 0).astype(np.int32)
        return attn_decode(q, kg, vg, eff, scale=scale, lib=lib)
    eff = np.where(active, ln, -1).astype(np.int32)   # -1: an inactive append row
    o, kg2, vg2 = attn_decode_append(q, k_new, v_new, kg, vg, eff, scale=scale, lib=lib)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in np.nonzero(active)[0]:
        kc2[rows[b]] = kg2[b]
        vc2[rows[b]] = vg2[b]
    return o, kc2, vc2


def attn_mixed(q, k, v, q_offset: int, qd, kcache, vcache, seqlens, *,
               scale: float | None = None, lib: ctypes.CDLL | None = None):
    """(O_chunk, O_decode) as float64 for a mixed batch of one layer.

    The batch holds a chunked-prefill chunk and single-token decode rows
    (kaispace.site note "Chunked Prefill"); each part is defined on its own:
    the chunk q[B,Hq,Nq,d] over k, v[B,Hkv,Nk,d] is the causal forward with
    query row i at position q_offset + i, and each decode row is the decode
    definition over its cache.  q is None: no chunk (None returned in its
    place); qd is None: no decode rows.  The default scale is 1/sqrt(d) of
    whichever part is present."""
    ref = q if q is not None else qd
    if ref is None:
        return None, None
    if scale is None:
        scale = 1.0 / np.sqrt(ref.shape[-1])
    o = None if q is None else attn_fwd(q, k, v, causal=True, q_offset=q_offset, scale=scale,
                                        lib=lib)
    od = None if qd is None else attn_decode(qd, kcache, vcache, seqlens, scale=scale, lib=lib)
    return o, od


def attn_bwd(q, k, v, dout, *, causal: bool = False, q_offset: int = 0,
             scale: float | None = None, lib: ctypes.CDLL | None = None):
    """(dQ, dK, dV) as float64 for a loss with dL/dO = dout: dQ has the shape
    of q [B,Hq,Nq,d]; dK, dV that of k and v [B,Hkv,Nk,d], each summed over
    the query heads that share the K/V head."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if do.shape != q.shape:
        raise ValueError("attn_bwd: dout must have the shape of q")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    _check(lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk),
                               _ptr(dv), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                               int(q_offset), float(scale)), "attn_bwd")
    return dq, dk, dv


def num_threads(lib: ctypes.CDLL | None = None) -> int:
    """OpenMP threads the oracle's parallel regions use in this process."""
    lib = lib or load()
    return int(lib.oracle_num_threads())
