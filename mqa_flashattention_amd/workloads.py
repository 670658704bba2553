"""Seeded synthetic inputs and the named workload shapes.

This module holds no attention arithmetic: it only draws inputs.  The tests
feed the same host tensors to the HIP library and to the CPU oracle, and the
benchmark draws its inputs here too.

Recipe (one torch CPU generator per draw, ``manual_seed(seed)``):
  forward: Q, K, V in that order, each ``torch.randn(shape, float32)``, i.e.
           N(0, 1); for bf16 workloads each tensor is then rounded to
           bfloat16 (round-to-nearest-even) -- the rounded values are the
           inputs both sides consume.
  decode:  q, K cache, V cache in that order as above, then the per-sequence
           cache lengths ``torch.randint(lo, hi + 1, (B,))`` (inclusive
           uniform integers) from the same generator.
  mixed:   the chunk as a forward draw with ``seed``, the decode rows as a
           decode draw with ``seed + 1``.
  varlen:  per-sequence lengths (when drawn) ``torch.randint(lo, hi + 1,
           (nseq,))`` from a generator seeded ``seed + 31``; then Q, K, V as
           the forward draw, token-major [total, H, d].

The shapes are the workloads the pages turn on:
  * LLaMA-3-8B attention shape (seq 2K, Hq 32, Hkv 8, d 128) from the
    BootstrapAI evolution log, "Kernel 9 -- GQA", KV-read estimate.
  * seq 4096 x 16 heads x batch 4 from the same log's "Kernel 8 --
    persistent kernel" scheduling example, with head dim 64 from its
    warp-specialization entry, swept over MHA / GQA / MQA (mode table of
    "Kernel 9").
  * cached decode at batch 8 with contexts up to 2048 (microLLM-rocm
    optimization log, experiments 060/085/294, which time steady decode at
    T2048 and B1..B8).
  * a 512-token chunk of a 4096-token prompt (kaispace.site note on Chunked
    Prefill, which splits a 4096-token prompt into chunks), alone and, as
    that note's mixed batch, beside decode rows of the same layer.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class FwdShape:
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool = False
    q_offset: int = 0
    dtype: torch.dtype = torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def visible_pairs_per_head(self) -> int:
        """Number of (query, key) pairs the causal mask leaves visible, per head."""
        if not self.causal:
            return self.Nq * self.Nk
        total = 0
        for i in range(self.Nq):
            total += min(self.Nk, self.q_offset + i + 1)
        return total


@dataclass(frozen=True)
class DecodeShape:
    B: int
    Hq: int
    Hkv: int
    Smax: int
    d: int
    len_lo: int
    len_hi: int
    dtype: torch.dtype = torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    fwd: tuple = field(default_factory=tuple)       # FwdShape variants
    decode: DecodeShape | None = None


WORKLOADS = {
    "tiny_gqa_f32": Workload(
        "tiny_gqa_f32",
        "Tiny GQA forward, fp32, non-causal: B=1 Hq=4 Hkv=2 N=64 d=32",
        fwd=(FwdShape(1, 4, 2, 64, 64, 32, False, 0, torch.float32),)),
    "llama3_8b_prefill": Workload(
        "llama3_8b_prefill",
        "LLaMA-3-8B-shaped causal prefill, bf16: B=1 Hq=32 Hkv=8 N=2048 d=128",
        fwd=(FwdShape(1, 32, 8, 2048, 2048, 128, True, 0),)),
    "mha_gqa_mqa_sweep": Workload(
        "mha_gqa_mqa_sweep",
        "MHA/GQA/MQA sweep, bf16, non-causal: B=4 N=4096 Hq=16 Hkv in {16,4,1} d=64",
        fwd=tuple(FwdShape(4, 16, hkv, 4096, 4096, 64, False, 0) for hkv in (16, 4, 1))),
    "kv_decode_b8": Workload(
        "kv_decode_b8",
        "KV-cache decode, bf16 cache: B=8 Hq=12 Hkv=2 d=128, lengths U[512,2048], Smax=2048",
        decode=DecodeShape(8, 12, 2, 2048, 128, 512, 2048)),
    "kv_decode_append_b8": Workload(
        "kv_decode_append_b8",
        "KV-cache decode with the new token's K/V appended in the same launch, bf16: B=8 Hq=12 "
        "Hkv=2 d=128, positions U[511,2047] (lengths U[512,2048] after the append), Smax=2048",
        decode=DecodeShape(8, 12, 2, 2048, 128, 512, 2048)),
    "chunked_prefill_4k": Workload(
        "chunked_prefill_4k",
        "Chunked prefill, bf16, causal: B=1 Hq=32 Hkv=8 d=128, Nq=512 at q_offset=3584, Nk=4096",
        fwd=(FwdShape(1, 32, 8, 512, 4096, 128, True, 3584),)),
    "llama3_8b_mixed": Workload(
        "llama3_8b_mixed",
        "Mixed batch in one launch, bf16, Hq=32 Hkv=8 d=128: the 512-query chunk at q_offset=3584 "
        "of a 4096-token prompt plus 8 decode rows, lengths U[512,4096], Smax=4096",
        fwd=(FwdShape(1, 32, 8, 512, 4096, 128, True, 3584),),
        decode=DecodeShape(8, 32, 8, 4096, 128, 512, 4096)),
    "llama3_8b_mixed_c128": Workload(
        "llama3_8b_mixed_c128",
        "The same mixed batch with a 128-query chunk (the prompt's last, q_offset=3968): fewer "
        "prefill units than CUs",
        fwd=(FwdShape(1, 32, 8, 128, 4096, 128, True, 3968),),
        decode=DecodeShape(8, 32, 8, 4096, 128, 512, 4096)),
}


def fwd_inputs(s: FwdShape, seed: int = 0):
    """CPU tensors (q, k, v) for a forward shape; see the module recipe."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((s.B, s.Hq, s.Nq, s.d), generator=g, dtype=torch.float32)
    k = torch.randn((s.B, s.Hkv, s.Nk, s.d), generator=g, dtype=torch.float32)
    v = torch.randn((s.B, s.Hkv, s.Nk, s.d), generator=g, dtype=torch.float32)
    return q.to(s.dtype), k.to(s.dtype), v.to(s.dtype)


def decode_inputs(s: DecodeShape, seed: int = 0):
    """CPU tensors (q, kcache, vcache, seqlens[int32]) for a decode shape."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((s.B, s.Hq, s.d), generator=g, dtype=torch.float32)
    kc = torch.randn((s.B, s.Hkv, s.Smax, s.d), generator=g, dtype=torch.float32)
    vc = torch.randn((s.B, s.Hkv, s.Smax, s.d), generator=g, dtype=torch.float32)
    lens = torch.randint(s.len_lo, s.len_hi + 1, (s.B,), generator=g, dtype=torch.int64)
    return q.to(s.dtype), kc.to(s.dtype), vc.to(s.dtype), lens.to(torch.int32)


def mixed_inputs(chunk: FwdShape, rows: DecodeShape, seed: int = 0):
    """CPU tensors (q, k, v, qd, kcache, vcache, seqlens) of a mixed batch:
    fwd_inputs(chunk, seed) then decode_inputs(rows, seed + 1)."""
    return (*fwd_inputs(chunk, seed), *decode_inputs(rows, seed + 1))


def append_inputs(s: DecodeShape, seed: int = 0):
    """CPU tensors (q, k_new, v_new, kcache, vcache, positions[int32]) for a
    decode-with-append step: q and the caches as decode_inputs(s, seed), the
    position of row b one less than its drawn length (so the row attends
    that many slots after the append), then the new K and V rows from their
    own generator seeded seed + 7919, in that order."""
    q, kc, vc, lens = decode_inputs(s, seed)
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    kn = torch.randn((s.B, s.Hkv, s.d), generator=g, dtype=torch.float32).to(s.dtype)
    vn = torch.randn((s.B, s.Hkv, s.d), generator=g, dtype=torch.float32).to(s.dtype)
    return q, kn, vn, kc, vc, (lens - 1).to(torch.int32)


@dataclass(frozen=True)
class VarlenShape:
    """A packed batch of nseq prompts, each a whole prompt (queries = keys),
    lengths uniform in [len_lo, len_hi]."""
    nseq: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int
    causal: bool = True
    dtype: torch.dtype = torch.bfloat16


# Prompts of mixed lengths batched into one prefill (microLLM-rocm
# optimization log, experiment 101, batches prompts of different lengths; the
# LLaMA-3-8B attention shape of the BootstrapAI log's "Kernel 9").
VARLEN_PREFILL = VarlenShape(nseq=8, Hq=32, Hkv=8, d=128, len_lo=128, len_hi=2048)


def varlen_lengths(s: VarlenShape, seed: int = 0) -> list[int]:
    g = torch.Generator(device="cpu").manual_seed(seed + 31)
    return [int(x) for x in torch.randint(s.len_lo, s.len_hi + 1, (s.nseq,), generator=g)]


def varlen_inputs(lens_q, lens_k, Hq: int, Hkv: int, d: int, dtype=torch.bfloat16,
                  seed: int = 0):
    """CPU tensors (q [sum lens_q, Hq, d], k and v [sum lens_k, Hkv, d],
    cu_seqlens_q, cu_seqlens_k [nseq + 1] int32) of a packed batch."""
    cq = torch.zeros(len(lens_q) + 1, dtype=torch.int32)
    ck = torch.zeros(len(lens_k) + 1, dtype=torch.int32)
    cq[1:] = torch.tensor(lens_q, dtype=torch.int64).cumsum(0).to(torch.int32)
    ck[1:] = torch.tensor(lens_k, dtype=torch.int64).cumsum(0).to(torch.int32)
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((int(cq[-1]), Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((int(ck[-1]), Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((int(ck[-1]), Hkv, d), generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype), cq, ck


def random_tensor(shape, seed: int, dtype=torch.float32, scale: float = 1.0):
    """One N(0, scale^2) tensor from its own seeded generator, rounded to dtype."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(dtype)
