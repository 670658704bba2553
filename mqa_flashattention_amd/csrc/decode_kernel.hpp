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
// The combine pass merges a row's partials (in a fixed order):
//   M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s acc_s / sum_s w_s l_s
// (m is kept in base-2 scaled units).  The fixed order makes the result
// bit-reproducible run to run.
//
// Decode with append (APPEND = true) folds the cache store of the new token
// into the same launch -- the K and V stores of one position done together
// (microLLM-rocm experiment 025) -- with a per-row position table (its
// experiments 083/084 and 098): row b's new K/V rows go to slot
// p = positions[b] and the row attends slots [0, p].  Only the split that
// holds slot p reads it, and that split takes the new rows straight from the
// inputs (patched into its staged LDS tile), so the store and the read of
// the slot need no ordering; its first column block performs the store.
#pragma once

#include "attn_tile.hpp"

namespace gqa {

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* seqlens;  // cached lengths; with append, the positions
  const void* knew;        // append: new K rows [B][Hkv][D]
  const void* vnew;        // append: new V rows [B][Hkv][D]
  void* kc_out;            // append: the K cache again, written at the positions
  void* vc_out;            // append: the V cache again
  void* o;
  float* ws;  // [B][Hq][NS][D + 4]: acc[D], m (scaled), l, 2 pad (16-byte records)
  // slot table: row b reads (and, appending, writes) cache row slots[b] of
  // Ncache; a slot outside [0, Ncache) marks an inactive row.  NULL: row b
  // is cache row b.
  const int32_t* slots;
  int Ncache;
  int B, Hq, Hkv, Smax;
  int g;      // Hq / Hkv
  int NCB;    // 32-head column blocks per K/V head, ceil(g / 32)
  int S_TOK;  // tokens per split (multiple of 32)
  int NS;     // splits per row, ceil(Smax / S_TOK)
  float c;    // |scale| * log2(e)
  float thr;  // kRescaleSlack / c
  int negate_q;
};

__device__ __forceinline__ int clamp_len(int32_t n, int smax) {
  return n < 0 ? 0 : (n > smax ? smax : n);
}

// Whether row b's slot (if there is a slot table) names a cache row.
__device__ __forceinline__ bool slot_ok(const DecodeArgs& a, int b) {
  if (!a.slots) return true;
  const int32_t s = a.slots[b];
  return s >= 0 && s < a.Ncache;
}

// Cache row of batch row b: its slot, or b without a slot table (0 for an
// inactive row, which reads and writes nothing).
__device__ __forceinline__ int cache_row(const DecodeArgs& a, int b) {
  if (!a.slots) return b;
  const int32_t s = a.slots[b];
  return (s >= 0 && s < a.Ncache) ? s : 0;
}

// Cache slots row b attends: the cached length clamped to [0, Smax]; with
// append, position p in [0, Smax) gives p + 1 (the new token included) and
// any other position marks an inactive row (0: no store, zero output), as
// does a slot outside the cache.
template <bool APPEND>
__device__ __forceinline__ int row_len(const DecodeArgs& a, int b) {
  if (!slot_ok(a, b)) return 0;
  const int32_t x = a.seqlens[b];
  if constexpr (APPEND) return (x >= 0 && x < a.Smax) ? x + 1 : 0;
  else return clamp_len(x, a.Smax);
}

// Overwrite key row r of a staged tile with a new row held as 16-byte
// chunks: lane c < D*ESZ/16 holds chunk c of the K row in kc and of the V
// row in vc.  K is row-major; V is row-major (fp32) or V^T[d][key] (bf16).
template <typename T, class C>
__device__ __forceinline__ void patch_row(T* __restrict__ Ks, T* __restrict__ Vs, int r, int c,
                                          const u32x4& kc, const u32x4& vc) {
  *reinterpret_cast<u32x4*>(Ks + r * C::KSTR + c * C::EPC) = kc;
  if constexpr (C::F32) {
    *reinterpret_cast<u32x4*>(Vs + r * C::VSTR + c * C::EPC) = vc;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      Vs[(8 * c + e) * C::VSTR + r] = (T)(vc[e >> 1] >> (16 * (e & 1)));
  }
}

// Orders one wave's LDS writes before its later LDS reads (and the reads
// before later writes).  WAVE: the wave runs alone in its LDS area while
// other waves of its workgroup do other work, so only the wave itself is
// ordered -- a wave's LDS operations complete in issue order, so keeping
// the compiler from moving them across this point is enough.  Otherwise a
// workgroup barrier (the workgroup is the one wave).
template <bool WAVE>
__device__ __forceinline__ void split_sync() {
  if constexpr (WAVE) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  } else {
    __syncthreads();
  }
}

// Split s_idx of row b for column block y = hkv * NCB + cb, run by one
// wavefront (lane 0..63) in the LDS area smem (C::STAGE_BYTES): reads the
// split's cache tiles, and writes its partial state for the combine pass.
template <typename T, class C, bool APPEND, bool WAVE>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, char* smem, int s_idx, int y,
                                             int b, int lane) {
  static_assert(C::NW == 1 && C::BC == 32, "decode works in single-wave 32-token tiles");
  T* const Ks = reinterpret_cast<T*>(smem);
  T* const Vs = Ks + C::K_ELEMS;

  const int hkv = y / a.NCB;
  const int cb = y % a.NCB;
  const int n = row_len<APPEND>(a, b);
  const int start = s_idx * a.S_TOK;
  if (start >= n) return;
  const int end = min(n, start + a.S_TOK);
  const int ntok = end - start;

  // append: the split holding the new token's slot (the row's last) loads
  // the new rows, stores them into the caches (first column block only) and
  // later patches them into the staged tile that holds the slot
  constexpr int CH = C::D * C::ESZ / 16;  // 16-byte chunks per row
  u32x4 nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
  int new_tile = -1, new_row = 0;
  if constexpr (APPEND) {
    if (end == n) {
      const int pos = n - 1;
      new_tile = (pos - start) / 32;
      new_row = (pos - start) % 32;
      if (lane < CH) {
        const size_t src = ((size_t)b * a.Hkv + hkv) * C::D;
        nk = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.knew) + src)[lane];
        nv = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.vnew) + src)[lane];
        if (cb == 0) {
          const size_t dst = (((size_t)cache_row(a, b) * a.Hkv + hkv) * a.Smax + pos) * C::D;
          reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.kc_out) + dst)[lane] = nk;
          reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.vc_out) + dst)[lane] = nv;
        }
      }
    }
  }
  const int j = lane & 31;
  const int h2 = lane >> 5;
  const int hig = cb * 32 + j;
  const bool valid = hig < a.g;
  const int h = hkv * a.g + hig;

  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q);
  typename C::Frag qf[C::QF];
  load_q_frag<T, C>(qf, Q + (valid ? ((size_t)b * a.Hq + h) * C::D : 0), valid,
                    a.negate_q != 0, h2);

  const size_t head_off = (((size_t)cache_row(a, b) * a.Hkv + hkv) * a.Smax + start) * C::D;
  const T* kbase = uniform_ptr(reinterpret_cast<const T*>(a.kc) + head_off);
  const T* vbase = uniform_ptr(reinterpret_cast<const T*>(a.vc) + head_off);

  float mrun = kNegInf, lrun = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  // Register stages: the loads of the next NSTG tiles are in flight while
  // tile t is computed.  Two in the decode kernel (one resident wave per
  // SIMD), so a split of up to two tiles costs one memory round trip; one
  // in a workgroup of the mixed kernel, whose register budget (two waves
  // per SIMD) holds one stage -- the same bytes in flight per SIMD.  With
  // two, the loop is unrolled by two so each stage is a named register set
  // (an indexed pair would be placed in scratch memory).
  constexpr int NSTG = WAVE ? 1 : 2;
  const int ntiles = (ntok + 31) / 32;
  TileRegs<C> ra, rb;
  load_tile<T, C>(ra, kbase, vbase, 0, ntok, lane, C::D * C::ESZ);
  if (NSTG > 1 && ntiles > 1) load_tile<T, C>(rb, kbase, vbase, 32, ntok, lane, C::D * C::ESZ);

  auto step = [&](TileRegs<C>& regs, int kt) {
    store_tile<T, C>(regs, Ks, Vs, lane);
    if constexpr (APPEND) {
      if (kt == new_tile && lane < CH) patch_row<T, C>(Ks, Vs, new_row, lane, nk, nv);
    }
    split_sync<WAVE>();
    if (kt + NSTG < ntiles)
      load_tile<T, C>(regs, kbase, vbase, (kt + NSTG) * 32, ntok, lane, C::D * C::ESZ);
    f32x16 s[C::KB];
    qk_tile<T, C>(s, qf, Ks, j, h2);
    const int key0 = kt * 32;
    if (key0 + 32 > ntok) mask_tile<C>(s, key0, ntok - 1, h2);
    softmax_pv_step<T, C>(s, mrun, lrun, acc, Vs, j, h2, a.c, a.thr);
    split_sync<WAVE>();
  };
  if constexpr (NSTG == 1) {
    for (int kt = 0; kt < ntiles; ++kt) step(ra, kt);
  } else {
    for (int kt = 0; kt < ntiles; kt += 2) {
      step(ra, kt);
      if (kt + 1 < ntiles) step(rb, kt + 1);
    }
  }

  const float lsum = halves_sum(lrun);
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

// grid (NS, Hkv * NCB, B), one wavefront per block.
template <typename T, class C, bool APPEND>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  decode_split<T, C, APPEND, false>(a, smem, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// grid (Hq, B), 256 threads.  Thread t takes 16-byte chunk t % (D/4) of
// the splits s = t / (D/4) (mod G).  When every thread has at most SPT
// splits (at d = 128: rows of up to 8 x 8 = 64 splits) it loads their
// maxima, sums and chunks in one memory round trip and keeps them in
// registers; otherwise the maxima are read first and the chunks in a second
// pass.  The G group sums are added through LDS in fixed order.
template <typename T, int D, bool APPEND>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  constexpr int REC = D + 4;    // floats per partial record
  constexpr int CH = D / 4;     // float4 chunks per record
  constexpr int G = 256 / CH;   // split groups
  constexpr int SPT = 8;        // splits per thread held in registers
  constexpr bool F32 = std::is_same<T, float>::value;
  __shared__ float s_red[4];
  __shared__ float4 s_acc[G][CH];
  __shared__ float s_l[G];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int n = row_len<APPEND>(a, b);
  T* orow = reinterpret_cast<T*>(a.o) + ((size_t)b * a.Hq + h) * D;
  if (n == 0) {
    for (int d = tid; d < D; d += 256) {
      if constexpr (F32) orow[d] = 0.f;
      else orow[d] = 0;
    }
    return;
  }
  const int ns = (n + a.S_TOK - 1) / a.S_TOK;
  const float* part = a.ws + ((size_t)b * a.Hq + h) * a.NS * REC;
  const int c = tid % CH;
  const int grp = tid / CH;

  // ---- M = max over splits of the scaled maxima (block-wide)
  auto block_max = [&](float mloc) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if ((tid & 63) == 0) s_red[tid >> 6] = mloc;
    __syncthreads();
    return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  };

  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (ns <= SPT * G) {
    // one round trip: everything this thread needs, then the reductions
    float m[SPT], l[SPT];
    float4 v[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int s = grp + k * G;
      m[k] = kNegInf;
      l[k] = 0.f;
      v[k] = float4{0.f, 0.f, 0.f, 0.f};
      if (s < ns) {
        const float* ps = part + (size_t)s * REC;
        v[k] = *reinterpret_cast<const float4*>(ps + 4 * c);
        m[k] = ps[D];
        l[k] = ps[D + 1];
      }
    }
    float mloc = m[0];
#pragma unroll
    for (int k = 1; k < SPT; ++k) mloc = fmaxf(mloc, m[k]);
    const float M = block_max(mloc);
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      // absent splits (m = -inf) weigh exactly 0
      const float wgt = fast_exp2(m[k] - M);
      acc.x += wgt * v[k].x;
      acc.y += wgt * v[k].y;
      acc.z += wgt * v[k].z;
      acc.w += wgt * v[k].w;
      L += wgt * l[k];
    }
  } else {
    float mloc = kNegInf;
    for (int s = tid; s < ns; s += 256) mloc = fmaxf(mloc, part[(size_t)s * REC + D]);
    const float M = block_max(mloc);
#pragma unroll 4
    for (int s = grp; s < ns; s += G) {
      const float* ps = part + (size_t)s * REC;
      const float wgt = fast_exp2(ps[D] - M);
      const float4 v = *reinterpret_cast<const float4*>(ps + 4 * c);
      acc.x += wgt * v.x;
      acc.y += wgt * v.y;
      acc.z += wgt * v.z;
      acc.w += wgt * v.w;
      L += wgt * ps[D + 1];
    }
  }
  s_acc[grp][c] = acc;
  if (c == 0) s_l[grp] = L;
  __syncthreads();
  if (tid < CH) {
    float4 t = s_acc[0][tid];
    float lt = s_l[0];
#pragma unroll
    for (int g2 = 1; g2 < G; ++g2) {
      const float4 u = s_acc[g2][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
      lt += s_l[g2];
    }
    const float inv = 1.0f / lt;
    if constexpr (F32) {
      *reinterpret_cast<float4*>(orow + 4 * tid) = float4{t.x * inv, t.y * inv, t.z * inv, t.w * inv};
    } else {
      *reinterpret_cast<u32x2*>(orow + 4 * tid) =
          u32x2{pack_bf16(t.x * inv, t.y * inv), pack_bf16(t.z * inv, t.w * inv)};
    }
  }
}

}  // namespace gqa
