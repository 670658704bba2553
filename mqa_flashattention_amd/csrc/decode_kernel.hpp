// decode_kernel.hpp -- single-token KV-cache decode: split-KV partials + combine.
//
// The cache of each sequence is cut into splits of S_TOK tokens (the
// split-sequence cached attention of the microLLM-rocm optimization log,
// experiments 283/284).  One wavefront owns one split of one K/V head and
// all g query heads that read it (up to 32, one MFMA column each), so each
// cache byte is read from HBM once and serves the whole group in place,
// without per-head copies (experiment 004 of the same log).  The wave walks
// its split in 32-token tiles with the same MFMA tile code as prefill --
// coalesced 16-byte cache loads staged through LDS, fp32 online softmax --
// and writes its partial state (running max m, sum l, unnormalised
// accumulator) to the workspace.  Splits past a row's length exit at once;
// the lengths live on the device and are read by the kernels.
//
// The combine pass merges a row's partials in split order:
//   M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s acc_s / sum_s w_s l_s
// (m is kept in base-2 scaled units).  The fixed order makes the result
// bit-reproducible run to run.
#pragma once

#include "attn_tile.hpp"

namespace gqa {

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* seqlens;
  void* o;
  float* ws;  // [B][Hq][NS][D + 4]: acc[D], m (scaled), l, 2 pad (16-byte records)
  int B, Hq, Hkv, Smax;
  int g;      // Hq / Hkv
  int NCB;    // 32-head column blocks per K/V head, ceil(g / 32)
  int S_TOK;  // tokens per split (multiple of 32)
  int NS;     // splits per row, ceil(Smax / S_TOK)
  float c;    // |scale| * log2(e)
  int negate_q;
};

__device__ __forceinline__ int clamp_len(int32_t n, int smax) {
  return n < 0 ? 0 : (n > smax ? smax : n);
}

// grid (NS, Hkv * NCB, B), one wavefront per block.
template <typename T, class C>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeArgs a) {
  static_assert(C::NW == 1 && C::BC == 32, "decode works in single-wave 32-token tiles");
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  T* const Ks = reinterpret_cast<T*>(smem);
  T* const Vs = Ks + C::K_ELEMS;

  const int s_idx = blockIdx.x;
  const int hkv = blockIdx.y / a.NCB;
  const int cb = blockIdx.y % a.NCB;
  const int b = blockIdx.z;
  const int n = clamp_len(a.seqlens[b], a.Smax);
  const int start = s_idx * a.S_TOK;
  if (start >= n) return;
  const int end = min(n, start + a.S_TOK);
  const int ntok = end - start;

  const int lane = threadIdx.x;
  const int j = lane & 31;
  const int h2 = lane >> 5;
  const int hig = cb * 32 + j;
  const bool valid = hig < a.g;
  const int h = hkv * a.g + hig;

  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q);
  typename C::Frag qf[C::QF];
  load_q_frag<T, C>(qf, Q + (valid ? ((size_t)b * a.Hq + h) * C::D : 0), valid,
                    a.negate_q != 0, h2);

  const size_t head_off = (((size_t)b * a.Hkv + hkv) * a.Smax + start) * C::D;
  const T* kbase = reinterpret_cast<const T*>(a.kc) + head_off;
  const T* vbase = reinterpret_cast<const T*>(a.vc) + head_off;

  float mrun = kNegInf, lrun = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const int ntiles = (ntok + 31) / 32;
  TileRegs<C> regs;
  load_tile<T, C>(regs, kbase, vbase, 0, ntok, lane);
  for (int kt = 0; kt < ntiles; ++kt) {
    store_tile<T, C>(regs, Ks, Vs, lane);
    __syncthreads();
    if (kt + 1 < ntiles) load_tile<T, C>(regs, kbase, vbase, (kt + 1) * 32, ntok, lane);

    f32x16 s[C::KB];
    qk_tile<T, C>(s, qf, Ks, j, h2);
    typename C::Frag pf[C::KB][C::PF];
    const int key0 = kt * 32;
    if (key0 + 32 > ntok)
      softmax_tile<C, true>(s, mrun, lrun, acc, pf, key0, ntok - 1, h2, a.c);
    else
      softmax_tile<C, false>(s, mrun, lrun, acc, pf, key0, ntok - 1, h2, a.c);
    pv_tile<T, C>(acc, pf, Vs, j, h2);
    __syncthreads();
  }

  const float lsum = lrun + __shfl_xor(lrun, 32);
  if (valid) {
    float* part = a.ws + (((size_t)b * a.Hq + h) * a.NS + s_idx) * (C::D + 4);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * h2;
        *reinterpret_cast<float4*>(part + d0) =
            float4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
      }
    }
    if (h2 == 0) {
      part[C::D] = mrun * a.c;
      part[C::D + 1] = lsum;
    }
  }
}

// grid (Hq, B), 64 threads; thread t produces d = t, t+64, ...
template <typename T, int D>
__global__ void __launch_bounds__(64) decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int n = clamp_len(a.seqlens[b], a.Smax);
  T* orow = reinterpret_cast<T*>(a.o) + ((size_t)b * a.Hq + h) * D;
  constexpr bool F32 = std::is_same<T, float>::value;
  if (n == 0) {
    for (int d = threadIdx.x; d < D; d += 64) {
      if constexpr (F32) orow[d] = 0.f;
      else orow[d] = 0;
    }
    return;
  }
  const int ns = (n + a.S_TOK - 1) / a.S_TOK;
  const float* part = a.ws + ((size_t)b * a.Hq + h) * a.NS * (D + 4);
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part[s * (D + 4) + D]);
  float L = 0.f;
  float accv[(D + 63) / 64];
#pragma unroll
  for (int u = 0; u < (D + 63) / 64; ++u) accv[u] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* ps = part + s * (D + 4);
    const float wgt = fast_exp2(ps[D] - M);
    L += wgt * ps[D + 1];
#pragma unroll
    for (int u = 0; u < (D + 63) / 64; ++u) {
      const int d = threadIdx.x + 64 * u;
      if (d < D) accv[u] += wgt * ps[d];
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int u = 0; u < (D + 63) / 64; ++u) {
    const int d = threadIdx.x + 64 * u;
    if (d < D) {
      const float x = accv[u] * inv;
      if constexpr (F32) {
        orow[d] = x;
      } else {
        orow[d] = (uint16_t)(pack_bf16(x, 0.f) & 0xffffu);
      }
    }
  }
}

}  // namespace gqa
