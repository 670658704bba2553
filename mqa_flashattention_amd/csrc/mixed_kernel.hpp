// mixed_kernel.hpp -- one launch for a mixed batch of one layer: the query
// chunk of a chunked prefill and single-token decode rows.
//
// Chunked prefill (kaispace.site note "Chunked Prefill") cuts a long prompt
// into chunks so that each step's batch holds a prompt chunk beside the
// decode tokens of other sequences.  Here both kinds of work come from one
// persistent launch (the work-queue scheduler of the BootstrapAI evolution
// log, "Kernel 8 -- persistent kernel", here with two kinds of item): a
// workgroup first takes the chunk's prefill units, heaviest first (or, with
// no more units than workgroups, runs the unit of its own index), and then
// takes decode work from one more counter: bf16, the parts of
// gqa_attn_decode, one per group of waves; fp32, splits, one per wave in an
// LDS area of its own.  So the decode work goes to the CUs that the prefill
// units leave idle -- at the start when the chunk has fewer units than
// resident workgroups, and in the tail.  The decode rows' partial states are
// merged by the decode merge (bf16) or combine (fp32) pass, launched after
// this kernel.
//
// Prefill and decode waves never share a CU: the prefill units use the
// whole register budget of two waves per SIMD.
//
// Three prefill shapes, as a prefill launch of the chunk would choose:
//  * mixed_kernel: 4-wave workgroups on 128-column units from the XCD
//    queues of the persistent schedule, for chunks with many units;
//  * mixed_quad_kernel: 8-wave workgroups on 64-column units whose keys
//    four 2-wave groups split (the quad schedule), for chunks with few,
//    long units -- a long chunk over a long prompt, where one wave walking
//    all of a unit's keys would be the critical path;
//  * mixed_balanced_kernel: the balanced schedule's equal chunks of key
//    tiles on part of the workgroups, for chunks with too few units to
//    balance whole ones (a short chunk over a long prompt, whose few units
//    would otherwise hold the launch while most CUs sit idle); the cut
//    units' partial states are merged after the launch.
#pragma once

#include <type_traits>

#include "decode_kernel.hpp"
#include "decode_part.hpp"
#include "prefill_kernel.hpp"

namespace gqa {

// Counter of the decode splits taken (after the prefill queues and the
// finished-workgroup count).
constexpr int kMixedDecodeCounter = kNumQueues + 1;
// LDS a mixed workgroup may use, so that two still fit on a CU.
constexpr int kMixedLdsBytes = 80 * 1024;
// Waves per bf16 decode part (one 16-column block; two blocks take half as
// many): the part kernel's, so that the records match gqa_attn_decode's.
#ifndef GQA_PART_W
#define GQA_PART_W 4
#endif
constexpr int kMixedPartW = GQA_PART_W;
// LDS of NWAVES waves' worth of bf16 decode parts.
template <int D, int NWAVES>
constexpr int mixed_part_lds_bytes() {
  constexpr int one = PartCfg<D, 1, kMixedPartW>::LDS_BYTES * (NWAVES / kMixedPartW);
  constexpr int two = PartCfg<D, 2, kMixedPartW / 2>::LDS_BYTES * (NWAVES / (kMixedPartW / 2));
  return one > two ? one : two;
}

struct MixedArgs {
  PrefillArgs p;  // the chunk (p.B == 0: none); p.ctr holds the counters
  DecodeArgs d;   // the decode rows
  int nd;         // decode splits, d.NS * d.Hkv * d.NCB * d.B (0: no decode rows)
};

// Waves of a workgroup that run decode splits: as many as have an LDS area
// of CD::STAGE_BYTES within kMixedLdsBytes.
template <class C, class CD>
constexpr int mixed_decode_waves() {
  constexpr int fit = kMixedLdsBytes / CD::STAGE_BYTES;
  return fit < 1 ? 1 : (fit < C::NW ? fit : C::NW);
}
template <class C, class CD>
constexpr int mixed_lds_bytes() {
  constexpr int pre = 2 * C::STAGE_BYTES;
  constexpr int dec = C::F32 ? mixed_decode_waves<C, CD>() * CD::STAGE_BYTES
                             : mixed_part_lds_bytes<C::D, C::NW>();
  return pre > dec ? pre : dec;
}

// Decode work, after the prefill units.  bf16: the parts of
// gqa_attn_decode (decode_part.hpp), each run by a group of P::W waves in an
// LDS area of its own -- the same records, so the same outputs, as a
// gqa_attn_decode call; take i covers parts DE*i .. DE*i + DE - 1 (DE =
// groups per workgroup), part x = (s, y, b) with s fastest, as the decode
// grid orders them.  fp32: DW waves (the LDS areas that fit) take one split
// each, staged through LDS (decode_split).  All threads of the workgroup
// call it.
template <class P>
__device__ __forceinline__ void mixed_part_takes(const MixedArgs& m, char* smem, int* s_take,
                                                 int nwaves) {
  const int tid = threadIdx.x;
  const int de = nwaves / P::W;
  const int grp = (tid >> 6) / P::W;
  const int ny = m.d.Hkv * m.d.NCB;
  for (;;) {
    __syncthreads();  // shared word read, LDS free of the previous part
    if (tid == 0) *s_take = atomicAdd(m.p.ctr + kMixedDecodeCounter * kCounterStride, 1);
    __syncthreads();
    const int take = __builtin_amdgcn_readfirstlane(*s_take);
    if ((long long)take * de >= m.nd) break;
    const int x = take * de + grp;
    const bool valid = grp < de && x < m.nd;
    const int xs = valid ? x : 0;
    const int s_idx = xs % m.d.NS;
    const int rest = xs / m.d.NS;
    // every group reaches the part's barrier, with work or without
    part_group<P, false>(m.d, smem + grp * P::LDS_BYTES, s_idx, rest % ny, rest / ny,
                         tid - grp * P::W * 64, valid);
  }
}

template <typename T, class CD, int DW, int NWAVES>
__device__ __forceinline__ void mixed_decode_phase(const MixedArgs& m, char* smem, int* s_take) {
  if constexpr (!std::is_same<T, float>::value) {
    if (m.d.g > 16)
      mixed_part_takes<PartCfg<CD::D, 2, kMixedPartW / 2>>(m, smem, s_take, NWAVES);
    else
      mixed_part_takes<PartCfg<CD::D, 1, kMixedPartW>>(m, smem, s_take, NWAVES);
  } else {
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ny = m.d.Hkv * m.d.NCB;
    for (;;) {
      __syncthreads();  // shared word read, LDS free of the previous item
      if (tid == 0) *s_take = atomicAdd(m.p.ctr + kMixedDecodeCounter * kCounterStride, 1);
      __syncthreads();
      const int take = __builtin_amdgcn_readfirstlane(*s_take);
      if ((long long)take * DW >= m.nd) break;
      const int x = take * DW + w;
      if (w < DW && x < m.nd) {
        const int s_idx = x % m.d.NS;
        const int rest = x / m.d.NS;
        decode_split<T, CD, false, true>(m.d, smem + w * CD::STAGE_BYTES, s_idx, rest % ny,
                                         rest / ny, lane);
      }
    }
  }
}

// Causal prefill units (config C) then decode splits (config CD); grid =
// resident workgroups (or fewer when there is less work).
template <typename T, class C, class CD>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
mixed_kernel(MixedArgs m) {
  constexpr int DW = mixed_decode_waves<C, CD>();
  __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<C, CD>()];
  static_assert(C::NW * stage_out_bytes<C>() <= 2 * C::STAGE_BYTES, "output staging too large");
  static_assert(C::D == CD::D, "one head dim for both parts");
  __shared__ int s_unit;
  __shared__ int s_queue;
  const PrefillArgs& a = m.p;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;

  // ---- prefill units (none without a chunk: no take at all)
  const int home = blockIdx.x % kNumQueues;
  const int nkv = a.B * a.Hkv;
  const int per_group = a.HB * a.NQB;
  bool home_empty = false;  // wave 0: the home queue has run dry
  for (; a.T > 0;) {
    __syncthreads();  // every wave has read the previous item's shared words
    if (w == 0) {
      int t, q;
      take_unit(a, home, nkv, per_group, home_empty, lane, t, q);
      if (lane == 0) {
        s_unit = t;
        s_queue = q;
      }
    }
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_unit);
    const int q = __builtin_amdgcn_readfirstlane(s_queue);
    if (t < 0) break;
    persistent_unit<T, C, true>(a, smem, t, q, w, j);
  }

  mixed_decode_phase<T, CD, DW, C::NW>(m, smem, &s_unit);
  leave_persistent(a, kMixedDecodeCounter);
}

// Causal chunk pieces of the balanced schedule (config C: workgroup g <
// nsl * Pp runs piece g, as prefill_balanced_kernel does), then decode work.
// The host sizes Pp for part of the resident workgroups, so the others start
// on the decode parts at once; the pieces' partial records are merged by
// the prefill merge pass after this kernel.
template <typename T, class C, class CD>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
mixed_balanced_kernel(MixedArgs m) {
  constexpr int DW = mixed_decode_waves<C, CD>();
  __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<C, CD>()];
  static_assert(C::NW * stage_out_bytes<C>() <= 2 * C::STAGE_BYTES, "output staging too large");
  static_assert(C::D == CD::D, "one head dim for both parts");
  __shared__ int s_take;
  if ((int)blockIdx.x < m.p.nsl * m.p.Pp) balanced_chunk<T, C, true>(m.p, smem, blockIdx.x);
  mixed_decode_phase<T, CD, DW, C::NW>(m, smem, &s_take);
  leave_persistent(m.p, kMixedDecodeCounter);
}

// Decode waves of a mixed_quad_kernel workgroup (8 waves, the quad
// schedule's LDS).
template <class CQ, class CD>
constexpr int mixed_quad_decode_waves() {
  constexpr int fit = quad_lds_bytes<CQ>() / CD::STAGE_BYTES;
  return fit < 1 ? 1 : (fit < 4 * CQ::NW ? fit : 4 * CQ::NW);
}

// Causal quad units (config CQ, 64 columns, m.p decomposed for them) from
// the persistent schedule's XCD queues (the units of a K/V group stay on one
// XCD, whose L2 then holds that group's K/V), heaviest position block first,
// then decode splits.
template <typename T, class CQ, class CD>
__global__ void __launch_bounds__(4 * CQ::NT) __attribute__((amdgpu_waves_per_eu(2)))
mixed_quad_kernel(MixedArgs m) {
  constexpr int DW = mixed_quad_decode_waves<CQ, CD>();
  constexpr int DEC = CQ::F32 ? DW * CD::STAGE_BYTES : mixed_part_lds_bytes<CQ::D, 4 * CQ::NW>();
  constexpr int LDS = quad_lds_bytes<CQ>() > DEC ? quad_lds_bytes<CQ>() : DEC;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  static_assert(CQ::D == CD::D, "one head dim for both parts");
  __shared__ int s_unit;
  __shared__ int s_queue;
  const PrefillArgs& a = m.p;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (a.T <= (int)gridDim.x) {
    // at most one unit per workgroup: workgroup i runs unit i as the quad
    // prefill launch maps it (a K/V group's units on one XCD), with no take
    if ((int)blockIdx.x < a.T) {
      const int i = blockIdx.x;
      const int t = (a.T % 8 == 0) ? (i % 8) * (a.T / 8) + i / 8 : i;
      quad_unit<T, CQ, true, false>(a, smem, t);
    }
    mixed_decode_phase<T, CD, DW, 4 * CQ::NW>(m, smem, &s_unit);
    leave_persistent(a, kMixedDecodeCounter);
    return;
  }
  const int home = blockIdx.x % kNumQueues;
  const int nkv = a.B * a.Hkv;
  const int per_group = a.HB * a.NQB;
  bool home_empty = false;  // wave 0: the home queue has run dry
  for (;;) {
    __syncthreads();  // shared words read, LDS free of the previous unit
    if (w == 0) {
      int t, q;
      take_unit(a, home, nkv, per_group, home_empty, lane, t, q);
      if (lane == 0) {
        s_unit = t;
        s_queue = q;
      }
    }
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_unit);
    const int q = __builtin_amdgcn_readfirstlane(s_queue);
    if (t < 0) break;
    // (queue, index) -> unit, as the persistent schedule maps causal units
    const int per_qb = (queue_units(q, nkv, per_group) / per_group) * a.HB;
    const int qb = a.NQB - 1 - t / per_qb;
    const int rest = t % per_qb;
    const int hb = rest % a.HB;
    const int kvg = q + kNumQueues * (rest / a.HB);
    quad_unit<T, CQ, true, false>(a, smem, (kvg * a.HB + hb) * a.NQB + qb);
  }
  mixed_decode_phase<T, CD, DW, 4 * CQ::NW>(m, smem, &s_unit);
  leave_persistent(a, kMixedDecodeCounter);
}

}  // namespace gqa
