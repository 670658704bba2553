// decode_part.hpp -- bf16 single-token KV-cache decode without LDS staging.
//
// The cache of row b, K/V head hkv is cut into parts of PT = W * TW * 32
// tokens (the split-sequence cached attention of the microLLM-rocm
// optimization log, experiments 283/284).  One workgroup of W waves takes
// one part for a group of up to 16 * NCB query heads of that K/V head (the
// head mapping hkv = h / g of the BootstrapAI evolution log, "Kernel 9"), so
// every cache byte is read from HBM once for the whole group, in place
// (experiment 004 of the microLLM-rocm log).  Wave w walks tiles w, w + W,
// ... of its part, 32 tokens each; the W partial states are merged through
// LDS and the workgroup writes one record (running max m, sum l,
// unnormalised accumulator) per query head; decode_combine_kernel merges a
// row's records.
//
// Everything inside a wave stays in registers.  Both contractions use
// v_mfma_f32_16x16x32_bf16 (16 rows x 16 columns x 32 deep): decode has at
// most a group's worth of queries, so 16 MFMA columns waste less than 32.
//   S^T = K Q^T : A = 16 key rows x 32 head dims, straight from global
//                 memory -- lane (r, q) of step t loads head dims
//                 32t + 8q .. +7 of key row rho(kb, r), so the four lanes of
//                 a row read 64 contiguous bytes per load instruction; B = the
//                 query fragment in the same head-dim order.
//   O^T = V^T P^T : A = 16 head dims x 32 keys.  Lane (r, q) loads
//                 16-byte pieces of 8 consecutive key rows (8 head dims each,
//                 4 full rows per load instruction) and transposes the 8 x 8
//                 block in registers with v_perm; output row i of MFMA db is
//                 head dim DPL*i + db.  B = the probabilities, which the
//                 score MFMA leaves in exactly the needed lanes: key row
//                 rho(kb, r) = 8*(r/4) + 4*kb + r%4 puts keys 8q .. 8q+7 of
//                 query n in lane (n, q).
// Per lane the output then holds D/4 contiguous head dims of one query.
//
// Online softmax in base 2 with the lazy reference of attn_tile.hpp: the
// running max is raised only when a tile exceeds it by kRescaleSlack / c;
// the probabilities are rounded to bf16 for the PV MFMA and l sums those
// rounded values.
#pragma once

#include "decode_kernel.hpp"

namespace gqa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Lane l and l ^ 16 combined in every lane (v_permlane16_swap with both
// operands x leaves x of the two 16-lane rows of each pair in the results).
__device__ __forceinline__ float rows16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Combined over the four lanes n, n+16, n+32, n+48 (one query's lanes).
__device__ __forceinline__ float quad_max(float x) { return halves_max(rows16_max(x)); }
__device__ __forceinline__ float quad_sum(float x) { return halves_sum(rows16_sum(x)); }

// Compile-time shape of the part kernel.
//   D   : head dim (32, 64, 128)
//   NCB : 16-query column blocks per wave (1 or 2)
//   W   : waves per workgroup
template <int D_, int NCB_, int W_>
struct PartCfg {
  static constexpr int D = D_;
  static constexpr int NCB = NCB_;
  static constexpr int W = W_;
  static constexpr int NT = 64 * W;
  static constexpr int DT = D / 32;   // 32-deep steps of the score MFMA
  static constexpr int DPL = D / 16;  // head dims per lane in a V row piece (= PV MFMAs)
  static constexpr int ROWB = D * 2;  // bytes per cache row
  static constexpr int COLS = 16 * NCB;
  static constexpr int RSTR = D + 4;  // floats per query row in the LDS merge area
  static constexpr int LDS_BYTES = W * COLS * RSTR * 4 + W * COLS * 8;
  // register stages of K/V tiles per wave: two (the next tile's loads in
  // flight during this one's compute) unless the accumulators of two column
  // blocks at d = 128 leave no room for a second set
  static constexpr int STAGES = D * NCB >= 256 ? 1 : 2;
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
};

// A V row piece of DPL bf16 (16, 8 or 4 bytes).
template <int DPL>
struct VPiece;
template <>
struct VPiece<8> {
  using type = u32x4;
  __device__ __forceinline__ static type load(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  }
  __device__ __forceinline__ static uint32_t word(const type& x, int i) { return x[i]; }
  __device__ __forceinline__ static type from_global(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
};
template <>
struct VPiece<4> {
  using type = u32x2;
  __device__ __forceinline__ static type load(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
  }
  __device__ __forceinline__ static uint32_t word(const type& x, int i) { return x[i]; }
  __device__ __forceinline__ static type from_global(const void* p) {
    return *reinterpret_cast<const u32x2*>(p);
  }
};
template <>
struct VPiece<2> {
  using type = uint32_t;
  __device__ __forceinline__ static type load(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  }
  __device__ __forceinline__ static uint32_t word(const type& x, int) { return x; }
  __device__ __forceinline__ static type from_global(const void* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
};

// MFMA row r of score block kb reads key row 8*(r/4) + 4*kb + r%4 of the tile.
__device__ __forceinline__ int part_key_row(int kb, int r) { return 8 * (r >> 2) + 4 * kb + (r & 3); }

// One tile's K and V as loaded: kr[kb][t] = key row part_key_row(kb, r),
// head dims 32t + 8q .. +7; vr[e] = key row 8q + e, head dims
// DPL*r .. DPL*r + DPL - 1.
template <class P>
struct PartTile {
  u32x4 kr[2][P::DT];
  typename VPiece<P::DPL>::type vr[8];
};

// Loads tile `tile` (keys 32*tile .. 32*tile + 31) of a part of ntok keys
// whose rows start at kbase / vbase, through buffer resources that start at
// the tile and cover only its rows below ntok: rows past the end read as
// zeros, and a tile wholly past the end costs no memory traffic (so a
// prefetch past the last tile can be issued unconditionally).  koff / voff:
// the lane's constant byte offsets.
template <class P>
__device__ __forceinline__ void part_load(PartTile<P>& x, const uint16_t* kbase,
                                          const uint16_t* vbase, int tile, int ntok, int koff0,
                                          int koff1, int voff) {
  const int key0 = tile * 32;
  const int rows = ntok - key0 < 32 ? (ntok - key0 > 0 ? ntok - key0 : 0) : 32;
  const uint64_t base = (uint64_t)(uint32_t)key0 * (uint32_t)P::ROWB;
  // uniform; readfirstlane keeps the resources in scalar registers
  const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)(rows * P::ROWB));
  const auto krs = buffer_rsrc(reinterpret_cast<const char*>(kbase) + base, bytes);
  const auto vrs = buffer_rsrc(reinterpret_cast<const char*>(vbase) + base, bytes);
#pragma unroll
  for (int t = 0; t < P::DT; ++t) {
    x.kr[0][t] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff0 + 64 * t, 0, 0);
    x.kr[1][t] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff1 + 64 * t, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x.vr[e] = VPiece<P::DPL>::load(vrs, voff + e * P::ROWB);
}

// The PV A operand for MFMA db: keys 8q .. 8q+7 of head dim DPL*r + db.
template <class P>
__device__ __forceinline__ bf16x8 part_vfrag(const PartTile<P>& x, int db) {
  using VP = VPiece<P::DPL>;
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = VP::word(x.vr[2 * i], db >> 1);
    const uint32_t b = VP::word(x.vr[2 * i + 1], db >> 1);
    w[i] = (db & 1) ? pair_hi(a, b) : pair_lo(a, b);
  }
  return __builtin_bit_cast(bf16x8, w);
}

// One wave's running state over some tiles of one segment (row b, K/V head
// hkv, column group cg): reference m (raw score units) and this lane's share
// l of the sum per column block, and the unnormalised O^T.
template <class P>
struct PartState {
  float m[P::NCB], l[P::NCB];
  f32x4 acc[P::NCB][P::DPL];
};

template <class P>
__device__ __forceinline__ void part_reset(PartState<P>& st) {
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb) {
    st.m[cb] = kNegInf;
    st.l[cb] = 0.f;
#pragma unroll
    for (int db = 0; db < P::DPL; ++db) st.acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// A segment: keys [start, start + ntok) of row b's cache, K/V head hkv,
// query column group cg; len is the row's length (with append: the new
// token is key len - 1).
struct PartSeg {
  int b, hkv, cg, start, ntok, len;
  int crow;               // the row's cache row (its slot)
  const uint16_t* kbase;  // key row `start` of the head, wave-uniform
  const uint16_t* vbase;
};

template <class P>
__device__ __forceinline__ PartSeg part_seg(const DecodeArgs& a, int b, int hkv, int cg,
                                            int start, int ntok, int len) {
  PartSeg sg;
  sg.b = b;
  sg.hkv = hkv;
  sg.cg = cg;
  sg.start = start;
  sg.ntok = ntok;
  sg.len = len;
  sg.crow = cache_row(a, b);
  const size_t head_off = (((size_t)sg.crow * a.Hkv + hkv) * a.Smax + start) * P::D;
  sg.kbase = uniform_ptr(reinterpret_cast<const uint16_t*>(a.kc) + head_off);
  sg.vbase = uniform_ptr(reinterpret_cast<const uint16_t*>(a.vc) + head_off);
  return sg;
}

// The raw query fragments of a segment's column group (loaded, not waited
// for): lane (n, q) of block cb holds head dims 32t + 8q .. +7 of query
// head cg * COLS + 16 cb + n of the group (a valid head's row for the
// columns past the group: their results are never stored).
template <class P>
__device__ __forceinline__ void part_q_load(const DecodeArgs& a, const PartSeg& sg,
                                            u32x4 (&qraw)[P::NCB][P::DT], int n, int q) {
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb) {
    const int hig = (sg.cg * P::NCB + cb) * 16 + n;
    const int h = sg.hkv * a.g + (hig < a.g ? hig : 0);
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)sg.b * a.Hq + h) * P::D;
#pragma unroll
    for (int t = 0; t < P::DT; ++t)
      qraw[cb][t] = *reinterpret_cast<const u32x4*>(qrow + 32 * t + 8 * q);
  }
}

// MFMA operands from the raw fragments; a negative scale is applied by
// negating Q (exact).
template <class P>
__device__ __forceinline__ void part_q_frag(const DecodeArgs& a,
                                            const u32x4 (&qraw)[P::NCB][P::DT],
                                            bf16x8 (&qf)[P::NCB][P::DT]) {
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb)
#pragma unroll
    for (int t = 0; t < P::DT; ++t) {
      u32x4 v = qraw[cb][t];
      if (a.negate_q) v ^= 0x80008000u;
      qf[cb][t] = __builtin_bit_cast(bf16x8, v);
    }
}

// One tile (segment keys 32*tile .. +31, staged in x) into the state.
template <class P, bool APPEND>
__device__ __forceinline__ void part_step(const DecodeArgs& a, const PartSeg& sg,
                                          PartState<P>& st, const bf16x8 (&qf)[P::NCB][P::DT],
                                          PartTile<P>& x, int tile, int lane) {
  const int n = lane & 15;
  const int q = lane >> 4;
  const float c = a.c;
  if constexpr (APPEND) {
    // the row's last slot (the new token) is taken from k_new / v_new
    const int new_key = sg.len - 1 - sg.start;
    if (sg.start + sg.ntok == sg.len && (new_key >> 5) == tile) {
      const int kr = new_key & 31;
      const size_t src = ((size_t)sg.b * a.Hkv + sg.hkv) * P::D;
      const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.knew) + src;
      const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.vnew) + src;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (part_key_row(kb, n) == kr) {
#pragma unroll
          for (int t = 0; t < P::DT; ++t)
            x.kr[kb][t] = *reinterpret_cast<const u32x4*>(kn + 32 * t + 8 * q);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * q + e == kr) x.vr[e] = VPiece<P::DPL>::from_global(vn + P::DPL * n);
      if (sg.cg == 0) {
        // store the new rows into the slot (16-byte chunks); every reader
        // of the slot takes it from k_new / v_new instead
        constexpr int CH = P::ROWB / 16;
        if (lane < CH) {
          const size_t dst =
              (((size_t)sg.crow * a.Hkv + sg.hkv) * a.Smax + sg.start + new_key) * P::D;
          reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.kc_out) + dst)[lane] =
              reinterpret_cast<const u32x4*>(kn)[lane];
          reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.vc_out) + dst)[lane] =
              reinterpret_cast<const u32x4*>(vn)[lane];
        }
      }
    }
  }

  // scores: s[cb][kb][i] = key 8q + 4kb + i of the tile, query n of block cb
  f32x4 s[P::NCB][2];
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < P::DT; ++t)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x.kr[kb][t]),
                                                     qf[cb][t], sc, 0, 0, 0);
      s[cb][kb] = sc;
    }
  const int key0 = tile * 32;
  if (key0 + 32 > sg.ntok) {
#pragma unroll
    for (int cb = 0; cb < P::NCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 8 * q + 4 * kb + i >= sg.ntok) s[cb][kb][i] = kNegInf;
  }
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb) {
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[cb][kb][i]);
    mt = quad_max(mt);
    if (__any(mt > st.m[cb] + a.thr)) {
      const float m_new = fmaxf(st.m[cb], mt);
      const float alpha = st.m[cb] == kNegInf ? 0.f : fast_exp2((st.m[cb] - m_new) * c);
      st.m[cb] = m_new;
      st.l[cb] *= alpha;
#pragma unroll
      for (int db = 0; db < P::DPL; ++db) st.acc[cb][db] *= alpha;
    }
    // weights against the reference, rounded to bf16; l sums the rounded values
    const float mc = st.m[cb] * c;
    u32x4 pw;
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float p0 = fast_exp2(__builtin_fmaf(s[cb][kb][2 * e], c, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(s[cb][kb][2 * e + 1], c, -mc));
        bf16x2 pk;
        pk.x = (__bf16)p0;
        pk.y = (__bf16)p1;
        float& la = e ? l1 : l0;
        la = __builtin_amdgcn_fdot2_f32_bf16(pk, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, la, false);
        pw[2 * kb + e] = __builtin_bit_cast(uint32_t, pk);
      }
    st.l[cb] += l0 + l1;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    // the V^T operands are transposed in registers just before their MFMA
#pragma unroll
    for (int db = 0; db < P::DPL; ++db)
      st.acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(part_vfrag<P>(x, db), pf,
                                                               st.acc[cb][db], 0, 0, 0);
  }
}

// Tiles first, first + step, ... below the segment's tile count into st.
// xa must already hold (or have in flight) the loads of tile `first`, and
// first must be a valid tile.  Two register stages when the budget allows
// (the next tile's loads in flight during this one's compute, unrolled by
// two so each stage is a named set); the prefetch is unconditional -- past
// the last tile it reads nothing -- so the wait before each step counts
// exactly the newer loads.
template <class P, bool APPEND>
__device__ __forceinline__ void part_walk(const DecodeArgs& a, const PartSeg& sg,
                                          PartState<P>& st, const bf16x8 (&qf)[P::NCB][P::DT],
                                          PartTile<P>& xa, PartTile<P>& xb, int first, int step,
                                          int ntiles, int lane, int koff0, int koff1, int voff) {
  if constexpr (P::STAGES == 1) {
    for (int t0 = first; t0 < ntiles; t0 += step) {
      if (t0 != first) {
        part_load<P>(xa, sg.kbase, sg.vbase, t0, sg.ntok, koff0, koff1, voff);
        __builtin_amdgcn_sched_barrier(0);
      }
      part_step<P, APPEND>(a, sg, st, qf, xa, t0, lane);
    }
  } else {
    for (int t0 = first; t0 < ntiles; t0 += 2 * step) {
      const int t1 = t0 + step;
      part_load<P>(xb, sg.kbase, sg.vbase, t1, sg.ntok, koff0, koff1, voff);
      __builtin_amdgcn_sched_barrier(0);
      part_step<P, APPEND>(a, sg, st, qf, xa, t0, lane);
      if (t1 >= ntiles) break;
      part_load<P>(xa, sg.kbase, sg.vbase, t1 + step, sg.ntok, koff0, koff1, voff);
      __builtin_amdgcn_sched_barrier(0);
      part_step<P, APPEND>(a, sg, st, qf, xb, t1, lane);
    }
  }
}

// Part `part` of row b for column y = hkv * NCB + cg, run by a group of
// P::W waves (group-relative thread gtid) in the LDS area smem
// (P::LDS_BYTES): its waves take interleaved tiles, their states are merged
// through LDS and the group writes one record per query head.  Every thread
// of the workgroup calls it at once -- it holds one workgroup barrier -- and
// a part at or past the row's length does nothing else.  APPEND: the part
// holding slot p = positions[b] takes that slot's K/V rows from k_new /
// v_new (its column group 0 also stores them in the caches).
template <class P, bool APPEND>
__device__ __forceinline__ void part_group(const DecodeArgs& a, char* smem, int part, int y,
                                           int b, int gtid, bool valid) {
  float* const acc_s = reinterpret_cast<float*>(smem);                      // [W][COLS][RSTR]
  float2* const ml_s = reinterpret_cast<float2*>(smem + P::W * P::COLS * P::RSTR * 4);  // [W][COLS]

  const int w = __builtin_amdgcn_readfirstlane(gtid >> 6);
  const int lane = gtid & 63;
  const int n = lane & 15;   // query column (score/output) or row r (A operands)
  const int q = lane >> 4;   // 16-lane row of the wave
  const int ncg = a.NCB;     // column groups of COLS queries per K/V head
  const int hkv = y / ncg;
  const int cg = y % ncg;

  const int len = valid ? row_len<APPEND>(a, b) : 0;
  const int start = part * a.S_TOK;
  const bool active = start < len;  // the merge pass ignores parts past the row's length
  const int ntok = active ? min(len - start, a.S_TOK) : 0;
  const int ntiles = (ntok + 31) >> 5;

  PartState<P> st;
  part_reset<P>(st);
  if (w < ntiles) {
    const PartSeg sg = part_seg<P>(a, b, hkv, cg, start, ntok, len);
    const int koff0 = part_key_row(0, n) * P::ROWB + 16 * q;
    const int koff1 = part_key_row(1, n) * P::ROWB + 16 * q;
    const int voff = 8 * q * P::ROWB + 2 * P::DPL * n;
    // the query fragments and the wave's first tile are requested together,
    // before anything waits for memory: one round trip after the length
    u32x4 qraw[P::NCB][P::DT];
    part_q_load<P>(a, sg, qraw, n, q);
    PartTile<P> xa, xb;
    part_load<P>(xa, sg.kbase, sg.vbase, w, ntok, koff0, koff1, voff);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 qf[P::NCB][P::DT];
    part_q_frag<P>(a, qraw, qf);
    part_walk<P, APPEND>(a, sg, st, qf, xa, xb, w, P::W, ntiles, lane, koff0, koff1, voff);
  }

  // ---- merge the W waves' states through LDS, then one record per query
  // lane (n, q) holds head dims (D/4)*q + j, j = DPL*rr + db, of query n
#pragma unroll
  for (int cb = 0; cb < P::NCB; ++cb) {
    const float lsum = quad_sum(st.l[cb]);
    float* row = acc_s + (w * P::COLS + cb * 16 + n) * P::RSTR + (P::D / 4) * q;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float v[P::DPL];
#pragma unroll
      for (int db = 0; db < P::DPL; ++db) v[db] = st.acc[cb][db][rr];
      if constexpr (P::DPL >= 4) {
#pragma unroll
        for (int k4 = 0; k4 < P::DPL / 4; ++k4)
          *reinterpret_cast<float4*>(row + P::DPL * rr + 4 * k4) =
              float4{v[4 * k4], v[4 * k4 + 1], v[4 * k4 + 2], v[4 * k4 + 3]};
      } else {
        *reinterpret_cast<float2*>(row + P::DPL * rr) = float2{v[0], v[1]};
      }
    }
    if (q == 0) ml_s[w * P::COLS + cb * 16 + n] = float2{st.m[cb], lsum};
  }
  __syncthreads();
  if (!active) return;
  // item i = (column qi, 16-byte chunk ch) of the merged state
  constexpr int CHN = P::D / 4;
  for (int i = gtid; i < P::COLS * CHN; i += P::NT) {
    const int qi = i / CHN;
    const int ch = i % CHN;
    const int hig = cg * P::COLS + qi;
    if (hig >= a.g) continue;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < P::W; ++v) M = fmaxf(M, ml_s[v * P::COLS + qi].x);
    float4 o = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < P::W; ++v) {
      const float2 mlv = ml_s[v * P::COLS + qi];
      // a wave without tiles (m = -inf) adds nothing
      const float wt = mlv.x == kNegInf ? 0.f : fast_exp2((mlv.x - M) * a.c);
      const float4 x = *reinterpret_cast<const float4*>(acc_s + (v * P::COLS + qi) * P::RSTR +
                                                        4 * ch);
      o.x += wt * x.x;
      o.y += wt * x.y;
      o.z += wt * x.z;
      o.w += wt * x.w;
      L += wt * mlv.y;
    }
    const int h = hkv * a.g + hig;
    float* rec = a.ws + (((size_t)b * a.Hq + h) * a.NS + part) * (P::D + 4);
    *reinterpret_cast<float4*>(rec + 4 * ch) = o;
    if (ch == 0) *reinterpret_cast<float2*>(rec + P::D) = float2{M * a.c, L};
  }
}

// grid (NP parts, Hkv * NCG column groups, B rows), P::NT threads: one part
// per workgroup.
template <class P, bool APPEND>
__global__ void __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(2)))
decode_part_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[P::LDS_BYTES];
  part_group<P, APPEND>(a, smem, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, true);
}

// Merges the part records of each (row b, query head h): grid (Hq, B), 256
// threads.  Thread t takes 16-byte chunk t % (D/4) of the parts
// s = t / (D/4) + k * G, k < 8 (G = 1024 / D groups; at most 8 * G parts).
// The row's length comes first; then every thread requests all of its
// records at once, with the part index clamped to the row's last part, so
// only records written by this call are read (the clamped repeats hit the
// caches) and the unused ones are dropped by selection.  The merge order is
// fixed (bit-reproducible):
//   M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s acc_s / sum_s w_s l_s.
template <int D, bool APPEND>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  constexpr int REC = D + 4;
  constexpr int CH = D / 4;
  constexpr int G = 256 / CH;
  constexpr int SPT = 8;
  __shared__ float s_red[4];
  __shared__ float4 s_acc[G][CH];
  __shared__ float s_l[G];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int c = tid % CH;
  const int grp = tid / CH;
  const float* part = a.ws + ((size_t)b * a.Hq + h) * a.NS * REC;

  const int n = row_len<APPEND>(a, b);
  const int ns = (n + a.S_TOK - 1) / a.S_TOK;
  const int last = ns > 0 ? ns - 1 : 0;
  float m[SPT], l[SPT];
  float4 v[SPT];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int s = min(grp + k * G, last);
    const float* ps = part + (size_t)s * REC;
    v[k] = *reinterpret_cast<const float4*>(ps + 4 * c);
    const float2 ml = *reinterpret_cast<const float2*>(ps + D);
    m[k] = ml.x;
    l[k] = ml.y;
  }
  float mloc = kNegInf;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    if (grp + k * G >= ns) {  // a repeat of the last part, or no part at all
      m[k] = kNegInf;
      l[k] = 0.f;
      v[k] = float4{0.f, 0.f, 0.f, 0.f};
    }
    mloc = fmaxf(mloc, m[k]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const float wgt = m[k] == kNegInf ? 0.f : fast_exp2(m[k] - M);
    acc.x += wgt * v[k].x;
    acc.y += wgt * v[k].y;
    acc.z += wgt * v[k].z;
    acc.w += wgt * v[k].w;
    L += wgt * l[k];
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
    // a row with no keys (n == 0) has no records: zero output
    const float inv = n > 0 ? 1.0f / lt : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + ((size_t)b * a.Hq + h) * D;
    *reinterpret_cast<u32x2*>(orow + 4 * tid) =
        u32x2{pack_bf16(t.x * inv, t.y * inv), pack_bf16(t.z * inv, t.w * inv)};
  }
}

}  // namespace gqa
