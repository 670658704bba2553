// attn_tile.hpp -- device building blocks of the gfx950 attention kernels.
//
// One wavefront owns 32 query columns.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32
// (fp32): K rows come from LDS as the A operand and the wave's Q fragment
// stays in registers as the B operand for the whole key loop.  In the 32x32
// accumulator layout a lane then holds 16 scores of ONE query (its column),
// so the row max and row sum of the online softmax are per-lane scalars plus
// a single exchange with the other half-wave.  The probabilities feed
// O^T = V^T P^T straight from registers as the B operand of the second MFMA;
// V is staged transposed in LDS so each lane's A operand is 16 contiguous
// bytes.  A fixed row permutation of K (bits 2 and 3 of the row index
// swapped) makes the keys a lane holds after the first MFMA exactly the 8
// contiguous keys the second MFMA wants, so nothing is shuffled between the
// two contractions.
//
// Online softmax: per tile, m' = max(m, rowmax s); alpha = 2^((m - m') c);
// p = 2^(s c - m' c); l' = alpha l + sum p; acc' = alpha acc + P V, with
// c = |scale| log2(e) -- the running-max rescale exp(m_old - m_new) of the
// tiled kernel in the BootstrapAI evolution log ("Kernel 2 -- tiling"),
// evaluated with the hardware base-2 exponential.  A negative scale is
// applied by negating Q (exact in bf16 and fp32) so c stays > 0; a zero
// scale is floored to a c so small that every weight rounds to exactly 1.
// In the bf16 path p is rounded to bf16 for the PV MFMA and l sums those
// same rounded values, so the normalisation matches the weights used.
//
// Accumulator layout of a 32x32 MFMA (CDNA3/CDNA4): lane L, register r holds
// row 8*(r/4) + 4*(L/32) + (r%4), column L%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even), first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Low / high 16-bit halves of two words, packed (a's half first): one
// v_perm_b32 each, whose selector picks bytes of {b, a} (a = bytes 0..3).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane l and lane l ^ 32 combined, in every lane: v_permlane32_swap with
// both operands x leaves (x[l mod 32], x[l mod 32 + 32]) in the two results,
// a VALU exchange of the half-waves instead of an LDS permute.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K row read by MFMA row i of a 32-key block: bits 2 and 3 of i swapped.
__device__ __forceinline__ int k_row_perm(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Key (within a 32-key block) held in accumulator register r by half-wave h2.
__device__ __forceinline__ constexpr int key_of_reg(int r, int h2) {
  return 16 * (r / 8) + 8 * h2 + (r % 8);
}

// Compile-time tile configuration.
//   T  : element type of Q/K/V/O (float or __bf16 stored as uint16)
//   D  : head dimension (32, 64, 128)
//   BC : keys per tile (multiple of 32)
//   NW : wavefronts sharing one K/V tile
//   KVS: K/V key rows at a run-time stride (token-major or padded layouts);
//        false: rows are contiguous, D elements apart (a compile-time stride,
//        so load offsets fold into the instructions)
template <typename T, int D_, int BC_, int NW_, bool KVS_ = false>
struct TileCfg {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int D = D_;
  static constexpr int BC = BC_;
  static constexpr int NW = NW_;
  static constexpr bool KVS = KVS_;
  static constexpr int NT = 64 * NW;
  static constexpr int KB = BC / 32;  // 32-key blocks per tile
  static constexpr int DB = D / 32;   // 32-row blocks of O^T
  static constexpr int ESZ = sizeof(T);
  static constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  // LDS: K row-major [BC][KSTR]; V row-major [BC][VSTR] (fp32) or V^T [D][VSTR] (bf16).
  static constexpr int KSTR = D + EPC;
  static constexpr int VSTR = F32 ? D + EPC : BC + EPC;
  static constexpr int K_ELEMS = BC * KSTR;
  static constexpr int V_ELEMS = F32 ? BC * VSTR : D * VSTR;
  static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * ESZ;
  // Global -> register staging in 16-byte chunks.
  static constexpr int ROW_CHUNKS = D / EPC;
  static constexpr int K_CHUNKS = BC * ROW_CHUNKS;
  static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  // bf16 V is transposed while staging: a thread takes VK consecutive keys of
  // one 8-element d-chunk and writes VK-key runs of 8 V^T rows.  Adjacent
  // threads take adjacent key groups of the same d-chunk, so one LDS write
  // instruction fills whole V^T rows (bank-conflict free with the padded
  // stride); each global load instruction still reads 64 contiguous bytes
  // per row.
  static constexpr int VK_RAW = K_CHUNKS / NT;
  static constexpr int VK = F32 ? 1 : (VK_RAW >= 8 ? 8 : (VK_RAW >= 4 ? 4 : (VK_RAW >= 2 ? 2 : 1)));
  static constexpr int KGROUPS = BC / VK;
  static constexpr int V_BLOCKS = KGROUPS * ROW_CHUNKS;
  static constexpr int V_PER_T = F32 ? K_PER_T : (V_BLOCKS + NT - 1) / NT;
  static constexpr int V_LOADS = F32 ? K_PER_T : V_PER_T * VK;
  // MFMA operand fragments of the wave's 32 queries.
  static constexpr int QF = F32 ? D / 2 : D / 16;
  using Frag = typename std::conditional<F32, float, bf16x8>::type;
  // Probabilities as the B operand of O^T = V^T P^T: fp32 -> one value per
  // MFMA (16 per key block); bf16 -> 8 values per MFMA (2 per key block).
  static constexpr int PF = F32 ? 16 : 2;

  static_assert(BC % 32 == 0, "tile must hold whole 32-key blocks");
  static_assert(D % 32 == 0, "head dim must be a multiple of 32");
  static_assert(BC % VK == 0, "V staging group must divide the tile");
};

template <class C>
struct TileRegs {
  u32x4 k[C::K_PER_T];
  u32x4 v[C::V_LOADS];
};

// p, declared wave-uniform (readfirstlane of both halves), so that values
// derived from it stay in scalar registers -- in particular the buffer
// resources below, which must be scalar.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// A raw buffer resource over `bytes` bytes at p.  Buffer loads at offsets at
// or beyond `bytes` return zeros without touching memory.  Stride 0; the
// third-dword value sets the 32-bit data-format field, which untyped buffer
// loads on this architecture need to be non-zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Issue the loads of one K/V tile -- keys key0 .. key0+BC-1 of one head
// whose rows start at kbase / vbase -- into registers, as 16-byte buffer
// loads through a resource that starts at row key0 and covers the rows below
// nkeys (at most one tile).  Rows at or beyond nkeys read as zeros; the
// caller masks those keys, so their weight is exactly 0.  The per-lane byte
// offsets do not depend on the tile, so the loop computes them once; the
// tile start is scalar work.  For K, consecutive threads take consecutive
// 16-byte chunks of a row, so a wave's load instruction covers whole rows.
// rowb: bytes from one key row to the next, a multiple of 16; used only when
// C::KVS (otherwise the rows are D * ESZ bytes apart).
// KPART false: V only (K staged another way; bf16).
template <typename T, class C, bool KPART = true>
__device__ __forceinline__ void load_tile(TileRegs<C>& r, const T* __restrict__ kbase,
                                          const T* __restrict__ vbase, int key0, int nkeys,
                                          int tid, int rowb) {
  static_assert(KPART || !C::F32, "V-only staging is bf16");
  const int ROWB = C::KVS ? rowb : C::D * C::ESZ;
  const int rows = nkeys - key0 < C::BC ? (nkeys - key0 > 0 ? nkeys - key0 : 0) : C::BC;
  // unsigned 32 x 32 -> 64-bit byte offset: scalar multiplies (a signed
  // 64-bit product would be done on the vector unit)
  const uint64_t base = (uint64_t)(uint32_t)key0 * (uint32_t)ROWB;
  // The range ends with the last existing row's last byte: (rows - 1) rows
  // apart, then one row of D elements.  For contiguous rows that is
  // rows * ROWB; for a token stride below a row's width (overlapping or
  // broadcast rows, stride 0 included) it still covers every row that
  // exists.  The range is uniform; readfirstlane keeps it (and so the
  // resource) in scalar registers -- a vector value here makes every load a
  // waterfall loop.
  const int span = rows > 0 ? (rows - 1) * ROWB + C::D * C::ESZ : 0;
  const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)span);
  const auto krs = buffer_rsrc(reinterpret_cast<const char*>(kbase) + base, bytes);
  const auto vrs = buffer_rsrc(reinterpret_cast<const char*>(vbase) + base, bytes);
#pragma unroll
  for (int n = 0; n < (KPART ? C::K_PER_T : 0); ++n) {
    const int id = tid + n * C::NT;
    if (C::K_CHUNKS % C::NT == 0 || id < C::K_CHUNKS) {
      const int row = id / C::ROW_CHUNKS;
      const int col = id % C::ROW_CHUNKS;
      const int off = row * ROWB + col * 16;
      r.k[n] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      if constexpr (C::F32) r.v[n] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    }
  }
  if constexpr (!C::F32) {
#pragma unroll
    for (int n = 0; n < C::V_PER_T; ++n) {
      const int id = tid + n * C::NT;
      if (C::V_BLOCKS % C::NT == 0 || id < C::V_BLOCKS) {
        const int kg = id % C::KGROUPS;
        const int dc = id / C::KGROUPS;
#pragma unroll
        for (int e = 0; e < C::VK; ++e)
          r.v[n * C::VK + e] =
              __builtin_amdgcn_raw_buffer_load_b128(vrs, (kg * C::VK + e) * ROWB + dc * 16, 0, 0);
      }
    }
  }
}

// Element i (0..7) of a 16-byte chunk of bf16, from VK chunks, packed as a
// VK-key run (first key in the lowest bits).
template <int VK>
struct VRun;
template <>
struct VRun<8> {
  using type = u32x4;
  __device__ __forceinline__ static type get(const u32x4* c, int i) {
    const int w = i >> 1;
    if (i & 1)
      return u32x4{pair_hi(c[0][w], c[1][w]), pair_hi(c[2][w], c[3][w]),
                   pair_hi(c[4][w], c[5][w]), pair_hi(c[6][w], c[7][w])};
    return u32x4{pair_lo(c[0][w], c[1][w]), pair_lo(c[2][w], c[3][w]),
                 pair_lo(c[4][w], c[5][w]), pair_lo(c[6][w], c[7][w])};
  }
};
template <>
struct VRun<4> {
  using type = u32x2;
  __device__ __forceinline__ static type get(const u32x4* c, int i) {
    const int w = i >> 1;
    if (i & 1) return u32x2{pair_hi(c[0][w], c[1][w]), pair_hi(c[2][w], c[3][w])};
    return u32x2{pair_lo(c[0][w], c[1][w]), pair_lo(c[2][w], c[3][w])};
  }
};
template <>
struct VRun<2> {
  using type = uint32_t;
  __device__ __forceinline__ static type get(const u32x4* c, int i) {
    const int w = i >> 1;
    return (i & 1) ? pair_hi(c[0][w], c[1][w]) : pair_lo(c[0][w], c[1][w]);
  }
};
template <>
struct VRun<1> {
  using type = uint16_t;
  __device__ __forceinline__ static type get(const u32x4* c, int i) {
    const int w = i >> 1;
    return (uint16_t)((i & 1) ? (c[0][w] >> 16) : (c[0][w] & 0xffffu));
  }
};

// Write a staged tile to LDS: K row-major; V row-major (fp32) or transposed
// (bf16, V^T[d][key]).
template <typename T, class C, bool KPART = true>
__device__ __forceinline__ void store_tile(const TileRegs<C>& r, T* __restrict__ Ks,
                                           T* __restrict__ Vs, int tid) {
#pragma unroll
  for (int n = 0; n < (KPART ? C::K_PER_T : 0); ++n) {
    const int id = tid + n * C::NT;
    if (C::K_CHUNKS % C::NT == 0 || id < C::K_CHUNKS) {
      const int row = id / C::ROW_CHUNKS;
      const int col = id % C::ROW_CHUNKS;
      *reinterpret_cast<u32x4*>(Ks + row * C::KSTR + col * C::EPC) = r.k[n];
      if constexpr (C::F32)
        *reinterpret_cast<u32x4*>(Vs + row * C::VSTR + col * C::EPC) = r.v[n];
    }
  }
  if constexpr (!C::F32) {
    using Run = VRun<C::VK>;
#pragma unroll
    for (int n = 0; n < C::V_PER_T; ++n) {
      const int id = tid + n * C::NT;
      if (C::V_BLOCKS % C::NT == 0 || id < C::V_BLOCKS) {
        const int kg = id % C::KGROUPS;
        const int dc = id / C::KGROUPS;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<typename Run::type*>(Vs + (dc * 8 + i) * C::VSTR + kg * C::VK) =
              Run::get(&r.v[n * C::VK], i);
      }
    }
  }
}

// ---- K staged by direct global -> LDS loads (bf16; d = 128 with 32-key
// tiles or d = 64 with 64-key tiles).  A K slot holds the tile's rows
// unpadded (D * 2 bytes each), with row r's 16-byte chunk c at chunk
// position c ^ f(r): a direct load writes the 16-byte chunks of a wave's 64
// lanes to 1 KiB of consecutive LDS (lane i at byte 16 i), which leaves no
// room for padding, and the XOR keeps the score MFMA's K fragment reads
// (rows 32 kb + k_row_perm(j), chunk 2 ks + h2) on distinct 16-byte bank
// groups: f(r) = r mod 16 for 256-byte rows, (r / 2) mod 8 for 128-byte
// rows (two rows per 256 bytes of banks).
template <class C>
constexpr bool direct_k_ok() {
  return !C::F32 && ((C::D == 128 && C::BC == 32) || (C::D == 64 && C::BC == 64));
}

template <class C>
constexpr int dk_slot_bytes() {
  return C::BC * C::D * 2;
}

template <class C>
__device__ __forceinline__ int dk_chunk_off(int row, int chunk) {
  if constexpr (C::D == 128) return row * 256 + ((chunk ^ (row & 15)) << 4);
  else return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Per-lane byte offsets of k_direct's loads within a tile (rows rowb bytes
// apart): wave w's instruction n fills the RPB rows of 1 KiB block
// n NW + w; lane i takes row RPB (n NW + w) + i / CPR at chunk position
// i % CPR, i.e. the row's chunk (i % CPR) ^ f(row).
template <class C>
struct KDirect {
  static constexpr int CPR = C::D / 8;               // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;               // rows per 1 KiB block
  static constexpr int NI = C::BC / RPB / C::NW;     // load instructions per thread
  static_assert((C::BC / RPB) % C::NW == 0, "whole 1 KiB blocks per wave");
  int off[NI];
};

template <class C>
__device__ __forceinline__ KDirect<C> k_direct_offsets(int tid, int rowb) {
  using K = KDirect<C>;
  const int ROWB = C::KVS ? rowb : C::D * 2;
  const int w = tid >> 6;
  const int i = tid & 63;
  K kd;
#pragma unroll
  for (int n = 0; n < K::NI; ++n) {
    const int r = K::RPB * (n * C::NW + w) + i / K::CPR;
    const int pos = i % K::CPR;
    // the chunk whose swizzled position is pos
    const int c = (dk_chunk_off<C>(r, pos) - r * (C::D * 2)) >> 4;
    kd.off[n] = r * ROWB + c * 16;
  }
  return kd;
}

// Issue the direct loads of tile rows key0 .. key0 + BC - 1 (below nkeys;
// rows past it are written as zeros) into slot Kd, at the lane offsets off
// (k_direct_offsets).  They complete in issue order with the wave's other
// vector-memory loads (one counter).
template <class C>
__device__ __forceinline__ void k_direct(const void* kbase, int key0, int nkeys, char* Kd, int tid,
                                         int rowb, const int* off) {
  static_assert(direct_k_ok<C>(), "direct K: bf16, d = 128 / 32-key or d = 64 / 64-key tiles");
  const int ROWB = C::KVS ? rowb : C::D * 2;
  const int rows = nkeys - key0 < C::BC ? (nkeys - key0 > 0 ? nkeys - key0 : 0) : C::BC;
  const uint64_t base = (uint64_t)(uint32_t)key0 * (uint32_t)ROWB;
  const int span = rows > 0 ? (rows - 1) * ROWB + C::D * 2 : 0;
  const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)span);
  const auto rs = buffer_rsrc(reinterpret_cast<const char*>(kbase) + base, bytes);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int n = 0; n < KDirect<C>::NI; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(Kd + (n * C::NW + w) * 1024), 16, off[n],
        0, 0, 0);
}

// The K chunks of a register-staged tile (load_tile's pattern) into slot Kd.
template <class C>
__device__ __forceinline__ void store_k_direct_layout(const TileRegs<C>& r, char* Kd, int tid) {
  static_assert(C::K_CHUNKS % C::NT == 0, "every thread holds whole K chunks");
#pragma unroll
  for (int n = 0; n < C::K_PER_T; ++n) {
    const int id = tid + n * C::NT;
    *reinterpret_cast<u32x4*>(Kd + dk_chunk_off<C>(id / C::ROW_CHUNKS, id % C::ROW_CHUNKS)) =
        r.k[n];
  }
}

// The wave's query fragment: column j of the B operand is query row qrow
// (for an invalid column the caller passes any valid row; its values are
// replaced by zero, so its scores are 0 and its output is dropped).  All
// loads are issued unconditionally, so they are in flight together.
template <typename T, class C>
__device__ __forceinline__ void load_q_frag(typename C::Frag (&qf)[C::QF],
                                            const T* __restrict__ qrow, bool valid,
                                            bool negate, int h2) {
#pragma unroll
  for (int ks = 0; ks < C::QF; ++ks) {
    if constexpr (C::F32) {
      const float x = qrow[2 * ks + h2];
      qf[ks] = valid ? (negate ? -x : x) : 0.f;
    } else {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h2);
      if (negate) w ^= 0x80008000u;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, valid ? w : zero);
    }
  }
}

// S^T for one tile: s[kb] holds keys 32*kb .. 32*kb+31 of the tile.
template <typename T, class C>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[C::KB], const typename C::Frag (&qf)[C::QF],
                                        const T* __restrict__ Ks, int lane32, int h2) {
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    f32x16 a = {};
    const T* krow = Ks + (32 * kb + k_row_perm(lane32)) * C::KSTR;
    if constexpr (C::F32) {
#pragma unroll
      for (int ks = 0; ks < C::QF; ++ks)
        a = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * ks + h2], qf[ks], a, 0, 0, 0);
    } else {
      // all K fragments are requested before the first MFMA (the scheduling
      // barrier keeps them there), so the LDS latency is paid once per block
      // instead of once per pair of MFMAs
      bf16x8 kf[C::QF];
#pragma unroll
      for (int ks = 0; ks < C::QF; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8*>(krow + 16 * ks + 8 * h2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < C::QF; ++ks)
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], a, 0, 0, 0);
    }
    s[kb] = a;
  }
}

// qk_tile over a K slot in the direct-load layout, from precomputed LDS
// addresses of slot 0's fragments (kp[kb][ks]: row 32 kb + k_row_perm(j),
// chunk 2 ks + h2); slot SL's lie SL * dk_slot_bytes further, a constant
// folded into the read instructions.
typedef __attribute__((address_space(3))) const char lds_cchar;
template <class C, int SL>
__device__ __forceinline__ void qk_tile_direct_at(f32x16 (&s)[C::KB], const bf16x8 (&qf)[C::QF],
                                                  lds_cchar* const (&kp)[C::KB][C::QF]) {
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    bf16x8 kf[C::QF];
#pragma unroll
    for (int ks = 0; ks < C::QF; ++ks)
      kf[ks] = *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
          kp[kb][ks] + SL * dk_slot_bytes<C>());
    __builtin_amdgcn_sched_barrier(0);
    f32x16 a = {};
#pragma unroll
    for (int ks = 0; ks < C::QF; ++ks)
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], a, 0, 0, 0);
    s[kb] = a;
  }
}

// ---- online softmax, one tile at a time (composed in softmax_pv_step).
// c must be > 0 (the host floors it), so masked scores (-inf) give weights
// of exactly 0.

// Exclude keys > lim of a tile starting at key key0 (scores set to -inf).
template <class C>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[C::KB], int key0, int lim, int h2) {
  const int rel = lim - key0 - 8 * h2;  // key_of_reg(r, h2) - 8*h2 <= rel  <=> visible
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * kb + 16 * (r / 8) + (r % 8) > rel) s[kb][r] = kNegInf;
}

// Row maximum of a tile's scores across both half-waves (each lane holds
// 16*KB scores of its query; the other half-wave holds the rest).
template <class C>
__device__ __forceinline__ float tile_rowmax(const f32x16 (&s)[C::KB]) {
  float mt = kNegInf;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[kb][r], s[kb][r + 1]));
  return halves_max(mt);
}

// Raise the running reference to m_new = max(m, mt) and rescale l and acc by
// alpha = 2^((m - m_new) c): 0 when m was -inf and m_new is finite, 1 while
// both are -inf (a lane whose keys so far were all masked has nothing
// accumulated yet).
template <class C>
__device__ __forceinline__ void raise_reference(float& m, float& l, f32x16 (&acc)[C::DB],
                                                float mt, float c) {
  const float m_new = fmaxf(m, mt);
  const float alpha = m_new == kNegInf ? 1.f : fast_exp2((m - m_new) * c);
  m = m_new;
  l *= alpha;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
}

// Weights p = 2^(s c - m c) of one tile against reference m, as the B operand
// of the PV MFMA; returns their sum (of the bf16-rounded values in the bf16
// path, via v_dot2_f32_bf16 against (1, 1)).
template <class C>
__device__ __forceinline__ float tile_weights(const f32x16 (&s)[C::KB], float m, float c,
                                              typename C::Frag (&pf)[C::KB][C::PF]) {
  const float mc = m == kNegInf ? 0.f : m * c;  // all-masked so far: every weight is 0
  float lt = 0.f, lt2 = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    if constexpr (C::F32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -mc));
        pf[kb][r] = p;
        lt += p;
      }
    } else {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * hk + 2 * e], c, -mc));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * hk + 2 * e + 1], c, -mc));
          bf16x2 pk;
          pk.x = (__bf16)p0;
          pk.y = (__bf16)p1;
          float& acc_l = (e & 1) ? lt2 : lt;  // two chains
          acc_l = __builtin_amdgcn_fdot2_f32_bf16(pk, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, acc_l,
                                                  false);
          w[e] = __builtin_bit_cast(uint32_t, pk);
        }
        pf[kb][hk] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
  return lt + lt2;
}

// acc[db] += V^T P^T for one tile (O^T rows 32*db .. 32*db+31).
template <typename T, class C>
__device__ __forceinline__ void pv_tile(f32x16 (&acc)[C::DB],
                                        const typename C::Frag (&pf)[C::KB][C::PF],
                                        const T* __restrict__ Vs, int lane32, int h2) {
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      if constexpr (C::F32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float vf = Vs[(32 * kb + key_of_reg(r, h2)) * C::VSTR + 32 * db + lane32];
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, pf[kb][r], acc[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              Vs + (32 * db + lane32) * C::VSTR + 32 * kb + 16 * hk + 8 * h2);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hk], acc[db], 0, 0, 0);
        }
      }
    }
  }
}

// One online-softmax + PV step on a (masked) score tile s:
//   if rowmax s exceeds m + thr in some lane (thr = kRescaleSlack / c, from
//   the host): m' = max(m, rowmax s), l and acc scaled by 2^((m - m') c);
//   p = 2^(s c - m c); l += sum p; acc += V^T P^T.
// The reference is raised only when needed (a wave-uniform branch; for
// m = -inf the bound m + thr is -inf, so the first tile with a visible key
// always raises it).  Between raises the weights are taken against a
// reference up to thr below the true running max, so they stay below
// 2^kRescaleSlack -- far inside fp32 and bf16 range -- and acc / l is
// unchanged in exact arithmetic.
constexpr float kRescaleSlack = 16.0f;

// The softmax half of the step: raises the reference if needed and leaves
// the weights in pf (for pv_tile) and their sum added to l.
template <class C>
__device__ __forceinline__ void softmax_step(const f32x16 (&s)[C::KB], float& m, float& l,
                                             f32x16 (&acc)[C::DB],
                                             typename C::Frag (&pf)[C::KB][C::PF], float c,
                                             float thr) {
  const float mt = tile_rowmax<C>(s);
  if (__any(mt > m + thr)) raise_reference<C>(m, l, acc, mt, c);
  l += tile_weights<C>(s, m, c, pf);
}

template <typename T, class C>
__device__ __forceinline__ void softmax_pv_step(f32x16 (&s)[C::KB], float& m, float& l,
                                                f32x16 (&acc)[C::DB], const T* __restrict__ Vs,
                                                int lane32, int h2, float c, float thr) {
  typename C::Frag pf[C::KB][C::PF];
  softmax_step<C>(s, m, l, acc, pf, c, thr);
  pv_tile<T, C>(acc, pf, Vs, lane32, h2);
}

// Store one query row of O from the O^T accumulator: this lane holds d =
// 32*db + 8*a + 4*h2 + (0..3) for a = 0..3.
template <typename T, class C>
__device__ __forceinline__ void store_out_block(T* __restrict__ orow, const f32x16& acc, float inv,
                                                int db, int h2) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int d0 = 32 * db + 8 * a + 4 * h2;
    const float x0 = acc[4 * a + 0] * inv;
    const float x1 = acc[4 * a + 1] * inv;
    const float x2 = acc[4 * a + 2] * inv;
    const float x3 = acc[4 * a + 3] * inv;
    if constexpr (C::F32) {
      *reinterpret_cast<float4*>(orow + d0) = float4{x0, x1, x2, x3};
    } else {
      *reinterpret_cast<u32x2*>(orow + d0) = u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
    }
  }
}

template <typename T, class C>
__device__ __forceinline__ void store_out_row(T* __restrict__ orow, const f32x16 (&acc)[C::DB],
                                              float inv, int h2) {
#pragma unroll
  for (int db = 0; db < C::DB; ++db) store_out_block<T, C>(orow, acc[db], inv, db, h2);
}

}  // namespace gqa
