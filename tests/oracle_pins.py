"""Pins for the CPU oracle: each checks it against something other than itself.

Used two ways:
  * ``tests/test_oracle.py`` runs every pin against the real oracle;
  * ``python tests/oracle_pins.py LIB.so`` runs them all against one compiled
    oracle library and exits non-zero if any fails.  ``test_oracle_mutants``
    uses that to show that a planted mistake in the oracle source (dropped
    term, wrong sign or index, transposed operand) fails at least one pin.

What pins what (each pin names the passage or mathematical fact it rests on):
  library    -- torch's scaled_dot_product_attention in fp64 on the CPU, with
                K/V heads replicated by repeat_interleave; for q_offset = 0 its
                own is_causal mask (top-left aligned) is used.  For the
                backward, torch autograd through the same routine.
  finite differences -- the backward against central differences of the
                (separately pinned) forward.
  closed forms and invariants -- see each function's docstring.
Inputs are numpy/torch draws with fixed seeds; nothing comes from the GPU.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

TOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _case(seed, B, Hq, Hkv, Nq, Nk, d):
    return (_rand((B, Hq, Nq, d), seed), _rand((B, Hkv, Nk, d), seed + 1),
            _rand((B, Hkv, Nk, d), seed + 2))


def _sdpa(q, k, v, causal, q_offset, scale):
    import torch
    import torch.nn.functional as F
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    Nq, Nk = qt.shape[2], kt.shape[2]
    if causal and q_offset == 0:
        out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    elif causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=(j <= q_offset + i),
                                             scale=scale)
    else:
        out = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out.numpy()


def _maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


# --------------------------------------------------------------------------- pins

def pin_library_attention(lib):
    """Whole definition vs a library attention routine (fp64) on random tiny shapes,
    MHA / GQA / MQA (BootstrapAI log, "Kernel 9" mode table), causal offsets
    0, 1, Nk-Nq and past the end."""
    rng = np.random.default_rng(1234)
    for t in range(24):
        Hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        Nq = int(rng.integers(1, 23))
        Nk = int(rng.integers(1, 29))
        d = int(rng.choice([4, 8, 32]))
        q, k, v = _case(100 + 3 * t, B, Hkv * g, Hkv, Nq, Nk, d)
        scale = 1.0 / math.sqrt(d)
        offsets = {0, 1, Nk + 3}
        if Nk >= Nq:
            offsets.add(Nk - Nq)
        for causal in (False, True):
            for off in (sorted(offsets) if causal else [0]):
                o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, scale=scale, lib=lib)
                ref = _sdpa(q, k, v, causal, off, scale)
                err = _maxerr(o, ref)
                assert err <= TOL, f"case {t} causal={causal} off={off}: err {err}"


def pin_decode_library(lib):
    """Decode vs the library routine on each row's first n cache slots."""
    rng = np.random.default_rng(77)
    for t in range(8):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 3, 6]))
        Smax = int(rng.integers(1, 40))
        d = int(rng.choice([8, 32]))
        q = _rand((B, Hkv * g, d), 500 + t)
        kc = _rand((B, Hkv, Smax, d), 600 + t)
        vc = _rand((B, Hkv, Smax, d), 700 + t)
        lens = rng.integers(1, Smax + 1, size=B).astype(np.int32)
        lens[0] = Smax
        scale = 1.0 / math.sqrt(d)
        o = oracle.attn_decode(q, kc, vc, lens, scale=scale, lib=lib)
        for b in range(B):
            n = int(lens[b])
            ref = _sdpa(q[b:b + 1, :, None, :], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n],
                        False, 0, scale)[0, :, 0, :]
            err = _maxerr(o[b], ref)
            assert err <= TOL, f"decode case {t} row {b}: err {err}"


def pin_gqa_equals_replicated_mha(lib):
    """GQA equals MHA with each K/V head repeated g times (consecutive query heads
    share a K/V head: h_kv = h_q / group_size)."""
    for causal, off in ((False, 0), (True, 0), (True, 5)):
        q, k, v = _case(11, 2, 8, 2, 13, 17, 8)
        o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, lib=lib)
        o_mha = oracle.attn_fwd(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                causal=causal, q_offset=off, lib=lib)
        assert np.array_equal(o, o_mha), "GQA != replicated MHA"


def pin_head_identity(lib):
    """V of K/V head t set to the constant t+1: query head h returns h//g + 1."""
    B, Hq, Hkv, N, d = 2, 12, 3, 9, 8
    q, k, _ = _case(21, B, Hq, Hkv, N, N, d)
    v = np.zeros((B, Hkv, N, d))
    for t in range(Hkv):
        v[:, t] = t + 1.0
    o = oracle.attn_fwd(q, k, v, causal=True, lib=lib)
    g = Hq // Hkv
    for h in range(Hq):
        assert np.all(np.abs(o[:, h] - (h // g + 1.0)) <= 1e-14), f"head {h}"


def pin_probs_sum_to_one(lib):
    """Each softmax row is a probability vector over its visible keys: weights
    >= 0, exactly zero where masked, summing to 1; and O = sum_j p_j v_j."""
    q, k, v = _case(31, 1, 4, 2, 10, 14, 8)
    for causal, off in ((False, 0), (True, 0), (True, 3)):
        o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, lib=lib)
        for h in range(4):
            for i in range(10):
                p = oracle.attn_probs(q, k, v, 0, h, i, causal=causal, q_offset=off, lib=lib)
                assert abs(p.sum() - 1.0) <= 1e-13
                assert np.all(p >= 0)
                if causal:
                    assert np.all(p[off + i + 1:] == 0.0)
                    assert np.all(p[:off + i + 1] > 0)
                assert _maxerr(p @ v[0, h // 2], o[0, h, i]) <= TOL


def pin_constant_v(lib):
    """Constant V returns that constant (softmax weights sum to one)."""
    q, k, _ = _case(41, 2, 4, 4, 11, 23, 8)
    v = np.full((2, 4, 23, 8), -1.75)
    for causal in (False, True):
        o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=2, lib=lib)
        assert np.all(np.abs(o + 1.75) <= 1e-14)


def pin_causal_row0(lib):
    """Causal with q_offset = 0: query row 0 sees only key 0, so it returns V[0]."""
    q, k, v = _case(51, 2, 6, 3, 7, 7, 8)
    o = oracle.attn_fwd(q, k, v, causal=True, q_offset=0, lib=lib)
    for h in range(6):
        assert np.array_equal(o[:, h, 0], v[:, h // 2, 0])


def pin_single_key(lib):
    """Nk = 1: every row returns V[0]."""
    q, k, v = _case(61, 1, 4, 1, 5, 1, 8)
    for causal in (False, True):
        o = oracle.attn_fwd(q, k, v, causal=causal, lib=lib)
        assert np.array_equal(o[0], np.broadcast_to(v[0, 0, 0], o[0].shape))


def pin_two_keys_closed_form(lib):
    """Two keys: O = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1."""
    from scipy.special import expit
    q, k, v = _case(71, 1, 2, 1, 6, 2, 8)
    scale = 0.3
    o = oracle.attn_fwd(q, k, v, scale=scale, lib=lib)
    for h in range(2):
        for i in range(6):
            s0 = scale * float(np.dot(q[0, h, i], k[0, 0, 0]))
            s1 = scale * float(np.dot(q[0, h, i], k[0, 0, 1]))
            ref = expit(s0 - s1) * v[0, 0, 0] + expit(s1 - s0) * v[0, 0, 1]
            assert _maxerr(o[0, h, i], ref) <= TOL


def pin_zero_scale_mean(lib):
    """scale = 0: uniform weights, so each row is the mean of its visible V rows."""
    q, k, v = _case(81, 1, 4, 2, 6, 9, 8)
    for causal, off in ((False, 0), (True, 0), (True, 2)):
        o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, scale=0.0, lib=lib)
        for h in range(4):
            for i in range(6):
                last = min(9, off + i + 1) if causal else 9
                ref = v[0, h // 2, :last].mean(axis=0)
                assert _maxerr(o[0, h, i], ref) <= TOL


def pin_key_shift_invariance(lib):
    """Adding one vector u to every key shifts a row's scores by scale*q.u, a
    row constant, which softmax cancels."""
    q, k, v = _case(91, 1, 4, 2, 8, 12, 8)
    u = _rand((8,), 92)
    for causal in (False, True):
        o1 = oracle.attn_fwd(q, k, v, causal=causal, lib=lib)
        o2 = oracle.attn_fwd(q, k + u, v, causal=causal, lib=lib)
        assert _maxerr(o1, o2) <= 1e-11


def pin_chunk_consistency(lib):
    """Chunked prefill: a chunk of queries at q_offset reproduces those rows of
    the full causal pass (kaispace.site note on Chunked Prefill)."""
    N, off, n = 30, 17, 9
    q, k, v = _case(101, 1, 4, 2, N, N, 8)
    full = oracle.attn_fwd(q, k, v, causal=True, lib=lib)
    part = oracle.attn_fwd(np.ascontiguousarray(q[:, :, off:off + n]), k, v, causal=True,
                           q_offset=off, lib=lib)
    assert _maxerr(full[:, :, off:off + n], part) <= 1e-14


def pin_offset_past_end_is_noncausal(lib):
    """q_offset >= Nk - 1 leaves every key visible: causal equals non-causal."""
    q, k, v = _case(111, 1, 2, 2, 5, 8, 8)
    a = oracle.attn_fwd(q, k, v, causal=False, lib=lib)
    for off in (7, 8, 100):
        b = oracle.attn_fwd(q, k, v, causal=True, q_offset=off, lib=lib)
        assert _maxerr(a, b) <= 1e-14


def pin_key_permutation(lib):
    """Non-causal attention does not depend on the order of the (key, value) pairs."""
    q, k, v = _case(121, 2, 4, 2, 7, 15, 8)
    perm = np.random.default_rng(5).permutation(15)
    a = oracle.attn_fwd(q, k, v, lib=lib)
    b = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], lib=lib)
    assert _maxerr(a, b) <= TOL


def pin_linearity_in_v(lib):
    """O is linear in V for fixed Q, K."""
    q, k, v1 = _case(131, 1, 4, 2, 6, 10, 8)
    v2 = _rand(v1.shape, 132)
    for causal in (False, True):
        a = oracle.attn_fwd(q, k, v1 + 2.0 * v2, causal=causal, lib=lib)
        b = oracle.attn_fwd(q, k, v1, causal=causal, lib=lib) + \
            2.0 * oracle.attn_fwd(q, k, v2, causal=causal, lib=lib)
        assert _maxerr(a, b) <= TOL


def pin_hardmax_limit(lib):
    """Very large scale: softmax tends to the one-hot of the largest score, so the
    row returns V at the argmax key (and stays finite, i.e. the max is
    subtracted before exponentiating)."""
    d, Nk = 8, 12
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, Nk, d))
    k[0, 0, :, 0] = np.linspace(-1.0, 1.0, Nk)[np.random.default_rng(3).permutation(Nk)]
    v = _rand((1, 1, Nk, d), 141)
    o = oracle.attn_fwd(q, k, v, scale=1e5, lib=lib)
    jmax = int(np.argmax(k[0, 0, :, 0]))
    assert np.all(np.isfinite(o))
    assert _maxerr(o[0, 0, 0], v[0, 0, jmax]) <= TOL


def pin_rows_match_full(lib):
    """The sampled-row entry computes the same rows as the full pass."""
    q, k, v = _case(151, 2, 6, 2, 9, 13, 8)
    full = oracle.attn_fwd(q, k, v, causal=True, q_offset=3, lib=lib)
    ids = np.array([0, 5, 17, 53, 107, 2 * 6 * 9 - 1])
    rows = oracle.attn_fwd_rows(q, k, v, ids, causal=True, q_offset=3, lib=lib)
    assert np.array_equal(rows, full.reshape(-1, 8)[ids])


def pin_decode_semantics(lib):
    """Decode = one query per row over the first n = clamp(seqlens, 0, Smax) slots;
    slots past n are never read (NaN there changes nothing); n = 0 gives zeros."""
    B, Hq, Hkv, Smax, d = 4, 6, 2, 19, 8
    q = _rand((B, Hq, d), 161)
    kc = _rand((B, Hkv, Smax, d), 162)
    vc = _rand((B, Hkv, Smax, d), 163)
    lens = np.array([1, 7, Smax, Smax + 5], dtype=np.int32)
    o = oracle.attn_decode(q, kc, vc, lens, lib=lib)
    for b in range(B):
        n = min(int(lens[b]), Smax)
        ref = oracle.attn_fwd(q[b:b + 1, :, None, :], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n],
                              lib=lib)[0, :, 0, :]
        assert _maxerr(o[b], ref) <= 1e-14
    kp, vp = kc.copy(), vc.copy()
    for b in range(B):
        kp[b, :, min(int(lens[b]), Smax):] = np.nan
        vp[b, :, min(int(lens[b]), Smax):] = np.nan
    assert np.array_equal(oracle.attn_decode(q, kp, vp, lens, lib=lib), o)
    z = oracle.attn_decode(q, kc, vc, np.array([0, -3, 1, 2], dtype=np.int32), lib=lib)
    assert np.all(z[0] == 0) and np.all(z[1] == 0)


def pin_mixed_decode_rows_are_chunk_rows(lib):
    """A chunked-prefill chunk and decode rows in one batch (kaispace.site note
    "Chunked Prefill"): the chunk's query at position p sees keys 0..p, and a
    decode row whose cache holds those keys (length p + 1) is that same query.
    So decode rows built from the chunk's own queries and keys reproduce the
    chunk's rows -- a causal diagonal, offset or length off by one, or a
    non-causal chunk, breaks this.  Each part absent leaves the other as its
    own definition."""
    Hq, Hkv, Nk, Nq, d = 6, 2, 37, 11, 16
    off = Nk - Nq
    q = _rand((1, Hq, Nq, d), 171)
    k = _rand((1, Hkv, Nk, d), 172)
    v = _rand((1, Hkv, Nk, d), 173)
    Smax = Nk + 5
    qd = np.ascontiguousarray(q[0].transpose(1, 0, 2))          # [Nq, Hq, d]
    kc = np.full((Nq, Hkv, Smax, d), np.nan)
    vc = np.full((Nq, Hkv, Smax, d), np.nan)
    kc[:, :, :Nk] = k[0]
    vc[:, :, :Nk] = v[0]
    lens = np.arange(off + 1, Nk + 1, dtype=np.int32)           # row i: position off + i
    o, od = oracle.attn_mixed(q, k, v, off, qd, kc, vc, lens, lib=lib)
    assert o.shape == q.shape and od.shape == qd.shape
    assert _maxerr(od, o[0].transpose(1, 0, 2)) <= 1e-13
    # the last row sees every key: the plain softmax over all Nk keys, by hand
    s = (k[0][np.arange(Hq) // (Hq // Hkv)] @ q[0, :, -1, :, None])[..., 0] / math.sqrt(d)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    last = (w[:, :, None] * v[0][np.arange(Hq) // (Hq // Hkv)]).sum(1) / w.sum(1, keepdims=True)
    assert _maxerr(o[0, :, -1], last) <= TOL
    o2, none_d = oracle.attn_mixed(q, k, v, off, None, None, None, None, lib=lib)
    assert none_d is None and np.array_equal(o2, o)
    none_c, od2 = oracle.attn_mixed(None, None, None, 0, qd, kc, vc, lens, lib=lib)
    assert none_c is None and np.array_equal(od2, od)


def _append_case(seed, B, Hkv, g, Smax, d):
    return (_rand((B, Hkv * g, d), seed), _rand((B, Hkv, d), seed + 1), _rand((B, Hkv, d), seed + 2),
            _rand((B, Hkv, Smax, d), seed + 3), _rand((B, Hkv, Smax, d), seed + 4))


def pin_append_library(lib):
    """Decode with append vs the library routine: row b attends the first pos cache slots
    followed by its new K/V row (n = pos + 1); the returned caches equal the inputs except
    slot pos of each K/V head of an active row, which holds the new rows; rows with
    pos < 0 or pos >= Smax are inactive (zero output, caches untouched)."""
    rng = np.random.default_rng(91)
    for t in range(8):
        B = int(rng.integers(3, 6))
        Hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 6]))
        Smax = int(rng.integers(2, 40))
        d = int(rng.choice([8, 32]))
        q, kn, vn, kc, vc = _append_case(900 + 10 * t, B, Hkv, g, Smax, d)
        pos = rng.integers(0, Smax, size=B).astype(np.int32)
        pos[0] = Smax - 1
        pos[1] = -1 - int(rng.integers(0, 3))
        pos[2] = Smax + int(rng.integers(0, 3))
        scale = 1.0 / math.sqrt(d)
        o, ko, vo = oracle.attn_decode_append(q, kn, vn, kc, vc, pos, scale=scale, lib=lib)
        for b in range(B):
            p = int(pos[b])
            if p < 0 or p >= Smax:
                assert np.all(o[b] == 0), f"case {t} row {b}: inactive row not zero"
                assert np.array_equal(ko[b], kc[b]) and np.array_equal(vo[b], vc[b])
                continue
            kk = np.concatenate([kc[b, :, :p], kn[b, :, None, :]], axis=1)
            vv = np.concatenate([vc[b, :, :p], vn[b, :, None, :]], axis=1)
            ref = _sdpa(q[b:b + 1, :, None, :], kk[None], vv[None], False, 0, scale)[0, :, 0, :]
            err = _maxerr(o[b], ref)
            assert err <= TOL, f"case {t} row {b}: err {err}"
            others = [j for j in range(Smax) if j != p]
            assert np.array_equal(ko[b][:, others], kc[b][:, others])
            assert np.array_equal(vo[b][:, others], vc[b][:, others])
            assert np.array_equal(ko[b][:, p], kn[b]) and np.array_equal(vo[b][:, p], vn[b])


def pin_append_first_slot(lib):
    """pos = 0: the query sees only its own new key, whose softmax weight is exactly 1,
    so every query head of K/V head hk returns v_new[b, hk] exactly."""
    B, Hkv, g, Smax, d = 3, 2, 3, 9, 16
    q, kn, vn, kc, vc = _append_case(171, B, Hkv, g, Smax, d)
    o, _, _ = oracle.attn_decode_append(q, kn, vn, kc, vc, np.zeros(B, np.int32), lib=lib)
    for h in range(Hkv * g):
        assert np.array_equal(o[:, h], vn[:, h // g]), f"head {h}"


def pin_append_equal_keys_mean(lib):
    """Every visible key equal to the new key: all scores tie, the weights are uniform,
    and the output is the mean of the pos cached V rows and the new V row."""
    B, Hkv, g, Smax, d = 4, 2, 2, 13, 8
    q, kn, vn, kc, vc = _append_case(181, B, Hkv, g, Smax, d)
    pos = np.array([3, 12, 7, 1], dtype=np.int32)
    for b in range(B):
        kc[b, :, :pos[b]] = kn[b, :, None, :]
    o, _, _ = oracle.attn_decode_append(q, kn, vn, kc, vc, pos, lib=lib)
    for b in range(B):
        p = int(pos[b])
        for h in range(Hkv * g):
            hk = h // g
            ref = (vc[b, hk, :p].sum(axis=0) + vn[b, hk]) / (p + 1)
            assert _maxerr(o[b, h], ref) <= 1e-12, f"row {b} head {h}"


# --------------------------------------------------------------------------- slot table

def _pool(seed, ncache, Hkv, Smax, d):
    return _rand((ncache, Hkv, Smax, d), seed), _rand((ncache, Hkv, Smax, d), seed + 1)


def pin_slots_library(lib):
    """Decode through a slot table vs the library routine on each row's own cache
    row: row b attends the first lengths[b] tokens of pool row slots[b] (rows may
    share a slot); appending, it attends pool row slots[b]'s first p tokens then
    its new K/V row, and the returned pools differ from the inputs exactly at
    position p of each active row's slot; a slot outside [0, Ncache) gives a
    zero row and touches nothing."""
    rng = np.random.default_rng(77)
    for t in range(6):
        ncache = int(rng.integers(5, 9))
        Hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 3]))
        Smax = int(rng.integers(3, 30))
        d = int(rng.choice([8, 16]))
        B = 5
        kc, vc = _pool(1100 + 10 * t, ncache, Hkv, Smax, d)
        q = _rand((B, Hkv * g, d), 1105 + 10 * t)
        slots = rng.permutation(ncache)[:B].astype(np.int32)
        slots[3] = -1 - int(rng.integers(0, 2))
        slots[4] = ncache + int(rng.integers(0, 2))
        scale = 1.0 / math.sqrt(d)
        # plain decode, one slot read by two rows
        plain = slots.copy()
        plain[1] = plain[0]
        lens = rng.integers(1, Smax + 1, size=B).astype(np.int32)
        o = oracle.attn_decode_slots(q, kc, vc, plain, lens, scale=scale, lib=lib)
        for b in range(B):
            sb = int(plain[b])
            if sb < 0 or sb >= ncache:
                assert np.all(o[b] == 0), f"case {t} row {b}: inactive row not zero"
                continue
            n = int(lens[b])
            ref = _sdpa(q[b:b + 1, :, None, :], kc[sb][None, :, :n], vc[sb][None, :, :n],
                        False, 0, scale)[0, :, 0, :]
            assert _maxerr(o[b], ref) <= TOL, f"case {t} row {b}"
        # append
        kn, vn = _rand((B, Hkv, d), 1107 + 10 * t), _rand((B, Hkv, d), 1108 + 10 * t)
        pos = rng.integers(0, Smax, size=B).astype(np.int32)
        o, ko, vo = oracle.attn_decode_slots(q, kc, vc, slots, pos, k_new=kn, v_new=vn,
                                             scale=scale, lib=lib)
        wk, wv = kc.copy(), vc.copy()
        for b in range(B):
            sb = int(slots[b])
            if sb < 0 or sb >= ncache:
                assert np.all(o[b] == 0), f"case {t} row {b}: inactive append row not zero"
                continue
            p = int(pos[b])
            kk = np.concatenate([kc[sb, :, :p], kn[b, :, None, :]], axis=1)
            vv = np.concatenate([vc[sb, :, :p], vn[b, :, None, :]], axis=1)
            ref = _sdpa(q[b:b + 1, :, None, :], kk[None], vv[None], False, 0, scale)[0, :, 0, :]
            assert _maxerr(o[b], ref) <= TOL, f"case {t} append row {b}"
            wk[sb, :, p] = kn[b]
            wv[sb, :, p] = vn[b]
        assert np.array_equal(ko, wk) and np.array_equal(vo, wv), f"case {t}: pools"


def pin_slots_identity(lib):
    """slots[b] = b over a pool of B rows is the plain batch, bit for bit."""
    B, Hkv, g, Smax, d = 4, 2, 2, 11, 8
    kc, vc = _pool(1200, B, Hkv, Smax, d)
    q = _rand((B, Hkv * g, d), 1202)
    lens = np.array([11, 0, 5, 1], dtype=np.int32)
    ident = np.arange(B, dtype=np.int32)
    assert np.array_equal(oracle.attn_decode_slots(q, kc, vc, ident, lens, lib=lib),
                          oracle.attn_decode(q, kc, vc, lens, lib=lib))
    kn, vn = _rand((B, Hkv, d), 1203), _rand((B, Hkv, d), 1204)
    pos = np.array([10, -1, 4, 0], dtype=np.int32)
    a = oracle.attn_decode_slots(q, kc, vc, ident, pos, k_new=kn, v_new=vn, lib=lib)
    b = oracle.attn_decode_append(q, kn, vn, kc, vc, pos, lib=lib)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def pin_slots_relabel(lib):
    """Moving the pool's rows to other places and relabelling the slot table to
    match changes nothing."""
    ncache, B, Hkv, g, Smax, d = 6, 4, 1, 4, 9, 8
    kc, vc = _pool(1300, ncache, Hkv, Smax, d)
    q = _rand((B, Hkv * g, d), 1302)
    slots = np.array([2, 5, 0, 3], dtype=np.int32)
    lens = np.array([9, 3, 7, 2], dtype=np.int32)
    o = oracle.attn_decode_slots(q, kc, vc, slots, lens, lib=lib)
    perm = np.array([4, 0, 5, 1, 3, 2])      # pool row r moves to place perm[r]
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    o2 = oracle.attn_decode_slots(q, kp, vp, perm[slots].astype(np.int32), lens, lib=lib)
    assert np.array_equal(o, o2)


# --------------------------------------------------------------------------- backward

def _sdpa_grads(q, k, v, dout, causal, q_offset, scale):
    """dQ, dK, dV by torch autograd (fp64) through its attention routine, K/V
    heads replicated by repeat_interleave -- whose own backward sums the
    replicas' gradients, i.e. the reduction over each K/V head's query heads."""
    import torch
    import torch.nn.functional as F
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True)
                  for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    kr, vr = kt.repeat_interleave(g, dim=1), vt.repeat_interleave(g, dim=1)
    Nq, Nk = qt.shape[2], kt.shape[2]
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= q_offset + i
    out = F.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask, scale=scale)
    out.backward(torch.from_numpy(np.ascontiguousarray(dout)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_bwd_library(lib):
    """dQ, dK, dV vs torch autograd through its attention routine (fp64) on
    random tiny shapes: MHA, GQA, MQA, causal offsets 0 / 1 / Nk-Nq / past the end."""
    cases = [(1, 2, 2, 5, 5, 4, False, 0), (2, 4, 2, 6, 9, 8, True, 3),
             (1, 6, 1, 7, 7, 8, True, 0), (1, 4, 4, 3, 8, 4, True, 5),
             (2, 8, 2, 4, 6, 4, True, 1), (1, 3, 1, 5, 4, 8, True, 9)]
    for n, (B, Hq, Hkv, Nq, Nk, d, causal, off) in enumerate(cases):
        q, k, v = _case(600 + n, B, Hq, Hkv, Nq, Nk, d)
        do = _rand(q.shape, 700 + n)
        sc = 0.7 / math.sqrt(d)
        got = oracle.attn_bwd(q, k, v, do, causal=causal, q_offset=off, scale=sc, lib=lib)
        want = _sdpa_grads(q, k, v, do, causal, off, sc)
        for a, b_ in zip(got, want):
            assert _maxerr(a, b_) <= 1e-11, (n, _maxerr(a, b_))


def pin_bwd_finite_differences(lib):
    """Each gradient vs central differences of L = sum(dout * O) computed with
    the forward oracle (pinned on its own), at random coordinates of q, k, v."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 5, 7, 4
    q, k, v = _case(810, B, Hq, Hkv, Nq, Nk, d)
    do = _rand(q.shape, 811)
    sc, off = 0.6, 2
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=True, q_offset=off, scale=sc, lib=lib)

    def loss(qq, kk, vv):
        o = oracle.attn_fwd(qq, kk, vv, causal=True, q_offset=off, scale=sc, lib=lib)
        return float(np.sum(do * o))

    rng = np.random.default_rng(812)
    h = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in grad.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-8 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def pin_bwd_closed_forms(lib):
    """Nk = 1: every weight is 1, so dQ = dK = 0 and dV = the sum of dout over
    the group's heads and rows.  scale = 0: weights are uniform over the
    visible keys, dQ = dK = 0 and dV[j] = sum over rows i seeing j of dout[i] / |J_i|."""
    B, Hq, Hkv, Nq, d = 2, 6, 2, 4, 8
    q, k, v = _case(820, B, Hq, Hkv, Nq, 1, d)
    do = _rand(q.shape, 821)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=False, scale=0.9, lib=lib)
    g = Hq // Hkv
    assert np.max(np.abs(dq)) <= TOL and np.max(np.abs(dk)) <= TOL
    want = do.reshape(B, Hkv, g, Nq, d).sum(axis=(2, 3))[:, :, None, :]
    assert _maxerr(dv, want) <= TOL
    Nk, off = 6, 1
    q, k, v = _case(822, B, Hq, Hkv, Nq, Nk, d)
    do = _rand(q.shape, 823)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=True, q_offset=off, scale=0.0, lib=lib)
    assert np.max(np.abs(dq)) <= TOL and np.max(np.abs(dk)) <= TOL
    want = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                n = min(Nk, off + i + 1)
                want[b, h // g, :n] += do[b, h, i] / n
    assert _maxerr(dv, want) <= TOL


def pin_bwd_key_sum_zero(lib):
    """Adding one vector to every key shifts a row's scores by a constant and
    leaves O unchanged, so the key gradients of each K/V head sum to zero."""
    q, k, v = _case(830, 2, 4, 2, 6, 9, 8)
    do = _rand(q.shape, 831)
    _, dk, _ = oracle.attn_bwd(q, k, v, do, causal=True, q_offset=2, scale=0.8, lib=lib)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-11


def pin_bwd_gqa_equals_replicated_mha(lib):
    """GQA backward = MHA backward on K/V heads replicated g times, with the
    replicas' dK, dV summed back (and the same dQ)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 6, 2, 5, 7, 4
    q, k, v = _case(840, B, Hq, Hkv, Nq, Nk, d)
    do = _rand(q.shape, 841)
    g = Hq // Hkv
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=True, q_offset=1, scale=0.5, lib=lib)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    dq2, dk2, dv2 = oracle.attn_bwd(q, kr, vr, do, causal=True, q_offset=1, scale=0.5, lib=lib)
    assert _maxerr(dq, dq2) <= TOL
    assert _maxerr(dk, dk2.reshape(B, Hkv, g, Nk, d).sum(axis=2)) <= TOL
    assert _maxerr(dv, dv2.reshape(B, Hkv, g, Nk, d).sum(axis=2)) <= TOL


# ---------------------------------------------------------------- packed varlen

def _varlen_case(seed, lens_q, lens_k, Hq, Hkv, d):
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    q = _rand((int(cq[-1]), Hq, d), seed)
    k = _rand((int(ck[-1]), Hkv, d), seed + 1)
    v = _rand((int(ck[-1]), Hkv, d), seed + 2)
    return q, k, v, cq, ck


VARLEN_CASES = [
    # (lens_q, lens_k, Hq, Hkv, d): ragged mixes, empty and one-token sequences,
    # more queries than keys (causal rows that see no key), no keys at all
    ([5, 0, 7, 1, 3], [9, 3, 3, 0, 3], 4, 2, 8),
    ([1, 1, 1], [1, 6, 2], 3, 3, 4),
    ([12], [12], 6, 2, 8),
    ([4, 9, 2], [17, 9, 11], 2, 1, 32),
]


def pin_varlen_library(lib):
    """Packed varlen vs the library attention routine on each sequence's own
    tensors, with the mask written out: query i of a sequence with Nq queries
    and Nk keys sees keys j <= Nk - Nq + i (its queries are its last Nq
    tokens); a row that sees no key is zero by definition."""
    import torch
    import torch.nn.functional as F
    for t, (lq, lk, Hq, Hkv, d) in enumerate(VARLEN_CASES):
        q, k, v, cq, ck = _varlen_case(700 + 5 * t, lq, lk, Hq, Hkv, d)
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            o = oracle.attn_fwd_varlen(q, k, v, cq, ck, causal=causal, scale=scale, lib=lib)
            for s in range(len(lq)):
                q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
                nq, nk = q1 - q0, k1 - k0
                if nq == 0:
                    continue
                want = np.zeros((nq, Hq, d))
                if nk > 0:
                    qt = torch.from_numpy(q[q0:q1].transpose(1, 0, 2).copy())
                    kt = torch.from_numpy(k[k0:k1].transpose(1, 0, 2).copy())
                    vt = torch.from_numpy(v[k0:k1].transpose(1, 0, 2).copy())
                    kt = kt.repeat_interleave(Hq // Hkv, dim=0)
                    vt = vt.repeat_interleave(Hq // Hkv, dim=0)
                    i = torch.arange(nq)[:, None]
                    j = torch.arange(nk)[None, :]
                    mask = (j <= nk - nq + i) if causal else torch.ones(nq, nk, dtype=torch.bool)
                    seen = mask.any(dim=1)
                    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
                    out = torch.where(seen[None, :, None], out, torch.zeros_like(out))
                    want = out.numpy().transpose(1, 0, 2)
                err = _maxerr(o[q0:q1], want)
                assert err <= TOL, f"case {t} seq {s} causal={causal}: err {err}"


def pin_varlen_sequence_independence(lib):
    """A sequence's rows depend on its own tokens only: redrawing every other
    sequence's queries, keys and values leaves them bit-identical."""
    lq, lk, Hq, Hkv, d = VARLEN_CASES[3]
    q, k, v, cq, ck = _varlen_case(900, lq, lk, Hq, Hkv, d)
    o = oracle.attn_fwd_varlen(q, k, v, cq, ck, causal=True, lib=lib)
    q2, k2, v2 = _rand(q.shape, 901), _rand(k.shape, 902), _rand(v.shape, 903)
    s = 1
    q2[cq[s]:cq[s + 1]] = q[cq[s]:cq[s + 1]]
    k2[ck[s]:ck[s + 1]] = k[ck[s]:ck[s + 1]]
    v2[ck[s]:ck[s + 1]] = v[ck[s]:ck[s + 1]]
    o2 = oracle.attn_fwd_varlen(q2, k2, v2, cq, ck, causal=True, lib=lib)
    assert np.array_equal(o[cq[s]:cq[s + 1]], o2[cq[s]:cq[s + 1]])
    assert not np.array_equal(o, o2)


def pin_varlen_reorder(lib):
    """Packing the sequences in reverse order reverses the output blocks."""
    lq, lk, Hq, Hkv, d = VARLEN_CASES[0]
    q, k, v, cq, ck = _varlen_case(950, lq, lk, Hq, Hkv, d)
    o = oracle.attn_fwd_varlen(q, k, v, cq, ck, causal=True, lib=lib)
    n = len(lq)
    rq = [q[cq[s]:cq[s + 1]] for s in reversed(range(n))]
    rk = [k[ck[s]:ck[s + 1]] for s in reversed(range(n))]
    rv = [v[ck[s]:ck[s + 1]] for s in reversed(range(n))]
    rcq = np.concatenate([[0], np.cumsum(lq[::-1])])
    rck = np.concatenate([[0], np.cumsum(lk[::-1])])
    ro = oracle.attn_fwd_varlen(np.concatenate(rq), np.concatenate(rk), np.concatenate(rv),
                                rcq, rck, causal=True, lib=lib)
    want = np.concatenate([o[cq[s]:cq[s + 1]] for s in reversed(range(n))])
    assert np.array_equal(ro, want)


def pin_varlen_full_prompt_row0(lib):
    """A sequence with as many queries as keys is a whole prompt: causal row 0
    returns V[0] of its own keys exactly, and its last row equals the
    non-causal pass over all its keys."""
    lq, lk, Hq, Hkv, d = VARLEN_CASES[2]
    q, k, v, cq, ck = _varlen_case(980, lq, lk, Hq, Hkv, d)
    o = oracle.attn_fwd_varlen(q, k, v, cq, ck, causal=True, lib=lib)
    g = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(o[0, h], v[0, h // g])
    full = oracle.attn_fwd_varlen(q, k, v, cq, ck, causal=False, lib=lib)
    assert _maxerr(o[-1], full[-1]) <= TOL


PINS = [
    pin_library_attention,
    pin_decode_library,
    pin_gqa_equals_replicated_mha,
    pin_head_identity,
    pin_probs_sum_to_one,
    pin_constant_v,
    pin_causal_row0,
    pin_single_key,
    pin_two_keys_closed_form,
    pin_zero_scale_mean,
    pin_key_shift_invariance,
    pin_chunk_consistency,
    pin_offset_past_end_is_noncausal,
    pin_key_permutation,
    pin_linearity_in_v,
    pin_hardmax_limit,
    pin_rows_match_full,
    pin_decode_semantics,
    pin_mixed_decode_rows_are_chunk_rows,
    pin_append_library,
    pin_append_first_slot,
    pin_append_equal_keys_mean,
    pin_slots_library,
    pin_slots_identity,
    pin_slots_relabel,
    pin_bwd_library,
    pin_bwd_finite_differences,
    pin_bwd_closed_forms,
    pin_bwd_key_sum_zero,
    pin_bwd_gqa_equals_replicated_mha,
    pin_varlen_library,
    pin_varlen_sequence_independence,
    pin_varlen_reorder,
    pin_varlen_full_prompt_row0,
]


def main(argv):
    lib = oracle.load(argv[1], build_if_missing=False)
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception as e:  # any failure (assertion, NaN, bad return) counts
            failed.append(f"{pin.__name__}: {type(e).__name__}: {e}")
    for f in failed:
        print("FAIL", f)
    print(f"{len(PINS) - len(failed)}/{len(PINS)} pins passed")
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
