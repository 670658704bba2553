// mixed_kernel.hpp -- one launch for a mixed batch of one layer: the query
// chunk of a chunked prefill and single-token decode rows.
//
// Chunked prefill (kaispace.site note "Chunked Prefill") cuts a long prompt
// into chunks so that each step's batch holds a prompt chunk beside the
// decode tokens of other sequences.  Here both kinds of work come from one
// persistent launch (the work-queue scheduler of the BootstrapAI evolution
// log, "Kernel 8 -- persistent kernel", whose queue holds two kinds of
// item): a workgroup first takes the chunk's prefill units from the XCD
// queues, heaviest first, exactly as the persistent prefill schedule does;
// once every prefill queue is empty it takes decode splits from one more
// counter, DW at a time (one per wave, each wave in an LDS area of its own).
// So the decode splits fill the CUs that the prefill units leave idle --
// at the start when the chunk has fewer units than resident workgroups, and
// in the tail.  The decode rows' partial states are merged by the decode
// combine pass, launched after this kernel.
#pragma once

#include "decode_kernel.hpp"
#include "prefill_kernel.hpp"

namespace gqa {

// Counter of the decode splits taken (after the prefill queues and the
// finished-workgroup count).
constexpr int kMixedDecodeCounter = kNumQueues + 1;
// LDS a mixed workgroup may use, so that two still fit on a CU.
constexpr int kMixedLdsBytes = 80 * 1024;

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
  constexpr int dec = mixed_decode_waves<C, CD>() * CD::STAGE_BYTES;
  return pre > dec ? pre : dec;
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

  // ---- prefill units
  const int home = blockIdx.x % kNumQueues;
  const int nkv = a.B * a.Hkv;
  const int per_group = a.HB * a.NQB;
  bool home_empty = false;  // wave 0: the home queue has run dry
  for (;;) {
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

  // ---- decode splits: take i covers splits DW*i .. DW*i + DW - 1, split
  // x = (s, y, b) with s fastest, as the decode grid orders them
  const int ny = m.d.Hkv * m.d.NCB;
  for (;;) {
    __syncthreads();  // shared words read, LDS free of the previous item
    if (tid == 0) s_unit = atomicAdd(a.ctr + kMixedDecodeCounter * kCounterStride, 1);
    __syncthreads();
    const int take = __builtin_amdgcn_readfirstlane(s_unit);
    if ((long long)take * DW >= m.nd) break;
    const int x = take * DW + w;
    if (w < DW && x < m.nd) {
      const int s_idx = x % m.d.NS;
      const int rest = x / m.d.NS;
      decode_split<T, CD, false, true>(m.d, smem + w * CD::STAGE_BYTES, s_idx, rest % ny,
                                       rest / ny, lane);
    }
  }
  leave_persistent(a, kMixedDecodeCounter);
}

}  // namespace gqa
