"""CPU tests of the oracle: its pins, the method's algebra, and planted mistakes.

No GPU and no HIP code is involved.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import oracle_pins
from tests.oracle_pins import PINS, _case, _maxerr

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def lib():
    oracle.compile_oracle()  # always the current source
    return oracle.load()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(lib, pin):
    pin(lib)


# ------------------------------------------------------------------ method algebra
# The GPU path evaluates the definition with the tiled online-softmax
# recurrence (running max m, rescale exp(m_old - m_new) of the running sum and
# accumulator; BootstrapAI evolution log, "Kernel 2 -- tiling") and, for
# decode, with split-KV partials merged by a combine pass (microLLM-rocm
# optimization log, split-sequence experiments 283/284 and split-PV 291/292).
# In exact arithmetic both equal the definition; these fp64 re-derivations,
# written here from those descriptions, check that the algebra the kernels
# use is the definition the oracle computes.

def _online_row(qrow, K, V, last, scale, tiles):
    m, l, acc = -np.inf, 0.0, np.zeros(V.shape[1])
    start = 0
    for t in tiles:
        stop = min(start + t, last + 1)
        if stop <= start:
            break
        s = scale * (K[start:stop] @ qrow)
        m_new = max(m, float(s.max()))
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ V[start:stop]
        m = m_new
        start = stop
    return acc / l


def _split_combine_row(qrow, K, V, n, scale, split):
    parts = []
    for s0 in range(0, n, split):
        s = scale * (K[s0:min(n, s0 + split)] @ qrow)
        m = float(s.max())
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ V[s0:min(n, s0 + split)]))
    M = max(m for m, _, _ in parts)
    w = [np.exp(m - M) for m, _, _ in parts]
    num = sum(wi * a for wi, (_, _, a) in zip(w, parts))
    den = sum(wi * l for wi, (_, l, _) in zip(w, parts))
    return num / den


def test_online_recurrence_equals_definition(lib):
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 11, 37, 8
    q, k, v = _case(201, B, Hq, Hkv, Nq, Nk, d)
    scale = 0.35
    for causal, off in ((False, 0), (True, 0), (True, 20)):
        o = oracle.attn_fwd(q, k, v, causal=causal, q_offset=off, scale=scale, lib=lib)
        for h in range(Hq):
            for i in range(Nq):
                last = min(Nk - 1, off + i) if causal else Nk - 1
                tiles = list(rng.integers(1, 9, size=Nk))
                r = _online_row(q[0, h, i], k[0, h // 2], v[0, h // 2], last, scale, tiles)
                assert _maxerr(r, o[0, h, i]) <= 1e-12


def test_split_combine_equals_definition(lib):
    B, Hq, Hkv, Smax, d = 3, 6, 1, 45, 8
    rng = np.random.default_rng(10)
    qd = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, Smax, d))
    vc = rng.standard_normal((B, Hkv, Smax, d))
    lens = np.array([1, 30, 45], dtype=np.int32)
    o = oracle.attn_decode(qd, kc, vc, lens, scale=0.4, lib=lib)
    for split in (1, 4, 7, 32, 64):
        for b in range(B):
            for h in range(Hq):
                r = _split_combine_row(qd[b, h], kc[b, 0], vc[b, 0], int(lens[b]), 0.4, split)
                assert _maxerr(r, o[b, h]) <= 1e-12


# ------------------------------------------------------------------ planted mistakes
# Each mutant is the oracle source with one plausible mistake.  It is compiled
# to a temporary library and the whole pin suite runs against it in a child
# process (so a mutant that crashes also counts as caught).  Every mutant
# must fail at least one pin.
MUTANTS = [
    ("head map tiles instead of repeats", "const long hk = h / g;", "const long hk = h % Hkv;", 1),
    ("decode head map tiles", "const long hk = h / g;", "const long hk = h % Hkv;", 2),
    ("causal diagonal excluded", "last = q_offset + i;", "last = q_offset + i - 1;", 1),
    ("q_offset ignored", "if (causal && q_offset + i < last) last = q_offset + i;",
     "if (causal && i < last) last = i;", 1),
    ("scale dropped", "scores[j] = scale * dot;", "scores[j] = dot;", 1),
    ("decode scale dropped", "scores[j] = scale * dot;", "scores[j] = dot;", 2),
    ("max not subtracted", "scores[j] = exp(scores[j] - m);", "scores[j] = exp(scores[j]);", 1),
    ("shift sign flipped", "scores[j] = exp(scores[j] - m);", "scores[j] = exp(m - scores[j]);", 1),
    ("normalisation dropped", "for (long c = 0; c < d; ++c) out[c] /= l;", "", 1),
    ("K transposed", "dot += qrow[c] * kbase[j * d + c];", "dot += qrow[c] * kbase[c * Nk + j];", 1),
    ("V transposed", "out[c] += e * vbase[j * d + c];", "out[c] += e * vbase[c * Nk + j];", 1),
    ("V from query head", "const double* vbase = v + (b * Hkv + hk) * Nk * d;",
     "const double* vbase = v + (b * Hkv + h % Hkv) * Nk * d;", 1),
    ("Q read token-major", "q + ((b * Hq + h) * Nq + i) * d", "q + ((b * Nq + i) * Hq + h) * d", 1),
    ("decode length off by one", "long n = seqlens[b];", "long n = seqlens[b] - 1;", 1),
    ("decode clamp missing", "if (n > Smax) n = Smax;", "", 1),
    ("probabilities not normalised", "probs[j] = (j <= last) ? scores[j] / l : 0.0;",
     "probs[j] = (j <= last) ? scores[j] : 0.0;", 1),
    ("append length excludes the new token", "lens[b] = active ? (int32_t)(pos + 1) : 0;",
     "lens[b] = active ? (int32_t)pos : 0;", 1),
    ("append slot off by one", "double* kdst = kc + ((b * Hkv + hk) * Smax + pos) * d;",
     "double* kdst = kc + ((b * Hkv + hk) * Smax + pos - 1) * d;", 1),
    ("new V not appended", "memcpy(vdst, vsrc, sizeof(double) * (size_t)d);", "", 1),
    ("new K/V of head 0 for every head", "const double* ksrc = knew + (b * Hkv + hk) * d;",
     "const double* ksrc = knew + b * Hkv * d;", 1),
    ("capacity boundary not checked", "const int active = pos >= 0 && pos < Smax;",
     "const int active = pos >= 0;", 1),
    ("backward: D term dropped", "const double ds = probs[j] * (dp[j] - D);",
     "const double ds = probs[j] * dp[j];", 1),
    ("backward: softmax Jacobian sign flipped", "const double ds = probs[j] * (dp[j] - D);",
     "const double ds = probs[j] * (D - dp[j]);", 1),
    ("backward: dK scale dropped", "dkbase[j * d + c] += scale * ds * qrow[c];",
     "dkbase[j * d + c] += ds * qrow[c];", 1),
    ("backward: dQ from V instead of K", "dqrow[c] += scale * ds * kbase[j * d + c];",
     "dqrow[c] += scale * ds * vbase[j * d + c];", 1),
    ("backward: dV weighted by dS", "dvbase[j * d + c] += probs[j] * dorow[c];",
     "dvbase[j * d + c] += ds * dorow[c];", 1),
    ("backward: only the group's first head reduced", "for (long r = 0; r < g; ++r) {",
     "for (long r = 0; r < 1; ++r) {", 1),
    ("backward: dP from K", "for (long c = 0; c < d; ++c) dot += dorow[c] * vbase[j * d + c];",
     "for (long c = 0; c < d; ++c) dot += dorow[c] * kbase[j * d + c];", 1),
]


def _mutate(src: str, old: str, new: str, occurrence: int) -> str:
    pos = -1
    for _ in range(occurrence):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r} (occurrence {occurrence})"
    return src[:pos] + new + src[pos + len(old):]


def test_real_oracle_passes_suite_in_child(lib, tmp_path):
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), oracle.LIBRARY],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, occ):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(_mutate(src, old, new, occ))
    mutant_lib = str(tmp_path / "libmutant.so")
    oracle.compile_oracle(str(mutant_src), mutant_lib, strict=False)
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), mutant_lib],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "2"})
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout}"


# Planted mistakes in the mixed batch's composition (Python, not C): each
# wrong attn_mixed must fail the mixed-batch pin.
def _mixed_noncausal(q, k, v, off, qd, kc, vc, lens, *, scale=None, lib=None):
    return (oracle.attn_fwd(q, k, v, causal=False, lib=lib),
            oracle.attn_decode(qd, kc, vc, lens, lib=lib))


def _mixed_offset_off_by_one(q, k, v, off, qd, kc, vc, lens, *, scale=None, lib=None):
    return (oracle.attn_fwd(q, k, v, causal=True, q_offset=off - 1, lib=lib),
            oracle.attn_decode(qd, kc, vc, lens, lib=lib))


def _mixed_lengths_short(q, k, v, off, qd, kc, vc, lens, *, scale=None, lib=None):
    return (oracle.attn_fwd(q, k, v, causal=True, q_offset=off, lib=lib),
            oracle.attn_decode(qd, kc, vc, np.asarray(lens) - 1, lib=lib))


def _mixed_decode_unscaled(q, k, v, off, qd, kc, vc, lens, *, scale=None, lib=None):
    return (oracle.attn_fwd(q, k, v, causal=True, q_offset=off, lib=lib),
            oracle.attn_decode(qd, kc, vc, lens, scale=1.0, lib=lib))


@pytest.mark.parametrize("wrong", [_mixed_noncausal, _mixed_offset_off_by_one,
                                   _mixed_lengths_short, _mixed_decode_unscaled],
                         ids=lambda f: f.__name__[1:])
def test_planted_mixed_mistake_is_caught(lib, monkeypatch, wrong):
    monkeypatch.setattr(oracle, "attn_mixed", wrong)
    with pytest.raises(Exception):
        oracle_pins.pin_mixed_decode_rows_are_chunk_rows(lib)


# Planted mistakes in the packed varlen composition (Python): each wrong
# attn_fwd_varlen must fail one of the varlen pins.
def _varlen_mutant(kind):
    def f(q, k, v, cu_q, cu_k, *, causal=False, scale=None, lib=None):
        q, k, v = oracle._f64(q), oracle._f64(k), oracle._f64(v)
        cq, ck = np.asarray(cu_q, dtype=np.int64), np.asarray(cu_k, dtype=np.int64)
        if kind == "keys from query offsets":
            ck = cq.copy()
            ck[-1] = min(ck[-1], k.shape[0])
            ck = np.minimum(ck, k.shape[0])
        d = q.shape[2]
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        o = np.zeros_like(q)
        for s in range(len(cq) - 1):
            q0, q1, k0, k1 = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
            if kind == "rows shifted by one" and s > 0:
                q0, q1 = q0 - 1, q1 - 1
            nq, nk = q1 - q0, k1 - k0
            if nq <= 0 or nk <= 0:
                continue
            qs = q[q0:q1].transpose(1, 0, 2)[None]
            ks = k[k0:k1].transpose(1, 0, 2)[None]
            vs = v[k0:k1].transpose(1, 0, 2)[None]
            if not causal:
                o[q0:q1] = oracle.attn_fwd(qs, ks, vs, scale=scale, lib=lib)[0].transpose(1, 0, 2)
                continue
            off = nk - nq
            if kind == "top-left alignment":
                off = 0
            first = max(0, -off)
            if kind == "keyless rows get the mean of V":
                o[q0:q0 + first] = vs[0].mean(axis=1).repeat(q.shape[1] // k.shape[1], 0)
            if first >= nq:
                continue
            os_ = oracle.attn_fwd(qs[:, :, first:], ks, vs, causal=True, q_offset=off + first,
                                  scale=scale, lib=lib)
            o[q0 + first:q1] = os_[0].transpose(1, 0, 2)
        return o
    f.__name__ = kind.replace(" ", "_")
    return f


VARLEN_MUTANTS = ["top-left alignment", "keys from query offsets", "rows shifted by one",
                  "keyless rows get the mean of V"]


@pytest.mark.parametrize("kind", VARLEN_MUTANTS)
def test_planted_varlen_mistake_is_caught(lib, monkeypatch, kind):
    monkeypatch.setattr(oracle, "attn_fwd_varlen", _varlen_mutant(kind))
    caught = False
    for pin in (oracle_pins.pin_varlen_library, oracle_pins.pin_varlen_sequence_independence,
                oracle_pins.pin_varlen_reorder, oracle_pins.pin_varlen_full_prompt_row0):
        try:
            pin(lib)
        except Exception:
            caught = True
    assert caught, f"varlen mutant '{kind}' passed every varlen pin"


# Planted mistakes in the slot-table composition (Python): each wrong
# attn_decode_slots must fail one of the slot pins.
def _slots_mutant(kind):
    real = oracle.attn_decode_slots

    def f(q, kcache, vcache, slots, lengths, *, k_new=None, v_new=None, scale=None, lib=None):
        sl = np.asarray(slots, dtype=np.int64).copy()
        if kind == "slot table ignored":
            sl = np.arange(len(sl))
            sl = np.minimum(sl, np.asarray(kcache).shape[0] - 1)
        if kind == "inactive rows read pool row 0":
            sl = np.where((sl >= 0) & (sl < np.asarray(kcache).shape[0]), sl, 0)
        res = real(q, kcache, vcache, sl.astype(np.int32), lengths, k_new=k_new, v_new=v_new,
                   scale=scale, lib=lib)
        if kind == "append writes row b of the pool" and k_new is not None:
            o, kc2, vc2 = res
            kc2, vc2 = oracle._f64(kcache).copy(), oracle._f64(vcache).copy()
            pos = np.asarray(lengths)
            for b in range(len(sl)):
                if 0 <= sl[b] < kc2.shape[0] and 0 <= pos[b] < kc2.shape[2] and b < kc2.shape[0]:
                    kc2[b, :, pos[b]] = oracle._f64(k_new)[b]
                    vc2[b, :, pos[b]] = oracle._f64(v_new)[b]
            res = (o, kc2, vc2)
        return res
    return f


SLOTS_MUTANTS = ["slot table ignored", "inactive rows read pool row 0",
                 "append writes row b of the pool"]


@pytest.mark.parametrize("kind", SLOTS_MUTANTS)
def test_planted_slots_mistake_is_caught(lib, monkeypatch, kind):
    monkeypatch.setattr(oracle, "attn_decode_slots", _slots_mutant(kind))
    caught = False
    for pin in (oracle_pins.pin_slots_library, oracle_pins.pin_slots_identity,
                oracle_pins.pin_slots_relabel):
        try:
            pin(lib)
        except Exception:
            caught = True
    assert caught, f"slot-table mutant '{kind}' passed every slot pin"


def test_pin_module_importable():
    assert len(oracle_pins.PINS) >= 15
