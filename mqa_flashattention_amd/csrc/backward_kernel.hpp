// backward_kernel.hpp -- attention backward: dQ, dK, dV with the K/V
// gradients reduced over the query heads of each K/V head.
//
// The backward boundary of the microLLM-rocm optimization log (experiment
// 044: QK, causal softmax, PV and the GQA head mapping under one
// forward/backward boundary, no T x T probabilities kept and no K/V head
// copies; experiments 051-054: each row's probabilities recomputed, the K/V
// gradients reduced over the heads sharing a K/V head).  With row
// statistics lse = m c + log2 l (base 2, scaled) and D = sum_c dO O:
//
//   P  = 2^(S c - lse)          dP = dO V^T          dS = P (dP - D)
//   dQ = scale dS K             dK = scale dS^T Q    dV = P^T dO
//
// Two kernels, both on the forward's MFMA tile code with the operands
// swapped around, no atomics, fixed summation order:
//  * bwd_dq_kernel: one 128-column unit of query rows (the forward's units:
//    the group's heads stacked over positions).  One pass over the unit's
//    key tiles forms S^T = K Q^T and dP^T = V dO^T and accumulates
//    dQ^T += K^T (E^T (dP^T - D)) with unnormalised weights E under the
//    forward's online softmax, normalised by l at the end.  It writes lse
//    and D of its rows for the second kernel.
//  * bwd_dkdv_kernel: 32 keys per wave of one K/V head.  The wave walks
//    the query tiles of every query head of the group (this is the GQA
//    reduction, done in registers), with S = Q K^T and dP = dO V^T, and
//    accumulates dV^T += dO^T P and dK^T += Q^T dS.  The query steps of a
//    key block are cut into up to kBwdQuerySplitMax parts, one workgroup
//    each, whose fp32 results bwd_merge_kernel adds in part order.
// Each staged tile is loaded from global memory once and written to LDS
// row-major (the A operand of S or S^T, or of dP) and transposed (the A
// operand of the contraction over its rows).  Where two such buffers fit
// (bf16), the next tile is written to the other one while this one is
// used, one barrier per step.
#pragma once

#include "prefill_kernel.hpp"

namespace gqa {

struct BwdArgs {
  PrefillArgs f;  // shapes, contiguous strides, the dQ kernel's unit decomposition, c
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* lse;  // [B][Hq][Nq]: m c + log2 l of each query row
  float* dd;   // [B][Hq][Nq]: D = sum_c dO O
  float* part;  // [qsplit][2][B][Hkv][Nk][D] fp32: dK, dV of each query part
  int qsplit;   // query parts per key block, 1 .. kBwdQuerySplitMax
  float scale;
};

// Each K/V key block's query range is cut into up to this many parts, one
// workgroup each, so that the first key blocks of a causal launch (which
// every query sees) do not serialise the kernel and small launches still
// fill the CUs; bwd_merge_kernel adds the parts' dK, dV in part order.
// With one part the kernel writes dK, dV itself.
constexpr int kBwdQuerySplitMax = 16;

// LDS buffers of staged tiles in the backward kernels: two (tile t + 1
// written while tile t is used) when they fit in half of a CU's LDS, so
// that two workgroups still share a CU; else one, written between two
// barriers.
template <class C>
constexpr int bwd_buffers() {
  return 4 * C::STAGE_BYTES <= 80 * 1024 ? 2 : 1;
}

// The rows of one staged tile (keys or queries key0 .. key0 + BC - 1 of one
// head) in registers, loaded once and written to LDS twice: row-major (the
// A operand of a score MFMA) and transposed (the A operand of a product
// over these rows).  The thread's 16-byte chunks follow the transposed
// store's pattern (store_tile's V part: VK consecutive rows of one column
// chunk; fp32: the row-major pattern, whose V layout is row-major too).
template <class C>
struct RowRegs {
  u32x4 c[C::V_LOADS];
};

template <class C>
__device__ __forceinline__ bool rowreg_valid(int tid, int i) {
  if constexpr (C::F32)
    return C::K_CHUNKS % C::NT == 0 || tid + i * C::NT < C::K_CHUNKS;
  else
    return C::V_BLOCKS % C::NT == 0 || tid + (i / C::VK) * C::NT < C::V_BLOCKS;
}

// Row and 16-byte column chunk of the thread's chunk i.
template <class C>
__device__ __forceinline__ void rowreg_pos(int tid, int i, int& row, int& col) {
  if constexpr (C::F32) {
    const int id = tid + i * C::NT;
    row = id / C::ROW_CHUNKS;
    col = id % C::ROW_CHUNKS;
  } else {
    const int id = tid + (i / C::VK) * C::NT;
    row = (id % C::KGROUPS) * C::VK + i % C::VK;
    col = id / C::KGROUPS;
  }
}

// Issue the loads of rows key0 .. key0 + BC - 1 below nrows of the head at
// base (rows rowb bytes apart when C::KVS, else D elements), through a
// buffer resource over the existing rows: rows past nrows read as zeros
// (load_tile's resource).
template <typename T, class C>
__device__ __forceinline__ void load_rows(RowRegs<C>& r, const T* __restrict__ base, int key0,
                                          int nrows, int tid, int rowb) {
  const int ROWB = C::KVS ? rowb : C::D * C::ESZ;
  const int rows = nrows - key0 < C::BC ? (nrows - key0 > 0 ? nrows - key0 : 0) : C::BC;
  const uint64_t off = (uint64_t)(uint32_t)key0 * (uint32_t)ROWB;
  const int span = rows > 0 ? (rows - 1) * ROWB + C::D * C::ESZ : 0;
  const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)span);
  const auto rs = buffer_rsrc(reinterpret_cast<const char*>(base) + off, bytes);
#pragma unroll
  for (int i = 0; i < C::V_LOADS; ++i) {
    if (rowreg_valid<C>(tid, i)) {
      int row, col;
      rowreg_pos<C>(tid, i, row, col);
      r.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * ROWB + col * 16, 0, 0);
    }
  }
}

// Row-major copy (stride KSTR), as store_tile writes K.
template <typename T, class C>
__device__ __forceinline__ void store_rows(const RowRegs<C>& r, T* __restrict__ Ks, int tid) {
#pragma unroll
  for (int i = 0; i < C::V_LOADS; ++i) {
    if (rowreg_valid<C>(tid, i)) {
      int row, col;
      rowreg_pos<C>(tid, i, row, col);
      *reinterpret_cast<u32x4*>(Ks + row * C::KSTR + col * C::EPC) = r.c[i];
    }
  }
}

// The copy store_tile writes for V: transposed (bf16) or row-major with
// stride VSTR (fp32).
template <typename T, class C>
__device__ __forceinline__ void store_rows_t(const RowRegs<C>& r, T* __restrict__ Vs, int tid) {
  if constexpr (C::F32) {
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      if (rowreg_valid<C>(tid, i)) {
        int row, col;
        rowreg_pos<C>(tid, i, row, col);
        *reinterpret_cast<u32x4*>(Vs + row * C::VSTR + col * C::EPC) = r.c[i];
      }
    }
  } else {
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
              Run::get(&r.c[n * C::VK], i);
      }
    }
  }
}

// Sum over this lane's elements of x * y (two B-operand fragments of one
// column); the other half-wave holds the rest of the row.
template <class C>
__device__ __forceinline__ float frag_dot(const typename C::Frag (&x)[C::QF],
                                          const typename C::Frag (&y)[C::QF]) {
  float s = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::QF; ++ks) {
    if constexpr (C::F32) {
      s += x[ks] * y[ks];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)x[ks][e] * (float)y[ks][e];
    }
  }
  return s;
}

// fp32 accumulator tile (16 values of one column per 32-row block) -> the
// B-operand fragments of the second MFMA, rounded to bf16 in the bf16 path
// (the packing of tile_weights).
template <class C>
__device__ __forceinline__ void to_frag(const f32x16 (&x)[C::KB],
                                        typename C::Frag (&pf)[C::KB][C::PF]) {
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    if constexpr (C::F32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pf[kb][r] = x[kb][r];
    } else {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16(x[kb][8 * hk + 2 * e], x[kb][8 * hk + 2 * e + 1]);
        pf[kb][hk] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
}

// grid (T), C::NT threads: one unit of the forward decomposition per
// workgroup.  Causal units are taken heaviest first (position blocks in
// descending order, all heads of a block together), so that the light
// units fill in behind the heavy ones instead of ending the launch.
template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(BwdArgs ba) {
  const PrefillArgs& a = ba.f;
  // buffers of staged key tiles, used in turn: buffer sg holds K row-major,
  // V row-major and K transposed (as store_tile lays them out)
  constexpr int BUF = (2 * C::K_ELEMS + C::V_ELEMS) * C::ESZ;
  constexpr int NBUF = 2 * BUF <= 80 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char smem[NBUF * BUF];
  auto Krow = [&](int sg) { return reinterpret_cast<T*>(smem + sg * BUF); };
  auto Vrow = [&](int sg) { return Krow(sg) + C::K_ELEMS; };
  auto Kt = [&](int sg) { return Krow(sg) + 2 * C::K_ELEMS; };
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  const int per_qb = a.T / a.NQB;  // units of one position block
  const int t = blockIdx.x;
  const int qb = CAUSAL ? a.NQB - 1 - t / per_qb : t % a.NQB;
  const int rest = CAUSAL ? t % per_qb : t / a.NQB;
  const int hb = rest % a.HB;
  const int kvg = rest / a.HB;
  const int hkv = kvg % a.Hkv;
  const int b = kvg / a.Hkv;
  const Column col = lane_column<C>(a, b, hkv, hb, qb, w, j);

  typename C::Frag qf[C::QF], dof[C::QF], of[C::QF];
  load_q_frag<T, C>(qf, reinterpret_cast<const T*>(a.q) + col.row_off, col.valid, false, h2);
  load_q_frag<T, C>(dof, reinterpret_cast<const T*>(ba.dout) + col.row_off, col.valid, false,
                    h2);
  load_q_frag<T, C>(of, reinterpret_cast<const T*>(ba.o) + col.row_off, col.valid, false, h2);
  const float Dv = halves_sum(frag_dot<C>(dof, of));

  const T* kbase;
  const T* vbase;
  kv_bases<T, C>(a, b, hkv, kbase, vbase);
  const int ntiles = unit_tiles<C, CAUSAL>(a, qb);
  const int full_lim = CAUSAL ? min(a.Nk, a.q_offset + qb * a.R + 1) : a.Nk;
  const int lim = (CAUSAL && col.valid) ? min(a.q_offset + col.i, a.Nk - 1) : a.Nk - 1;
  const float c = a.c;

  // ---- one pass over the unit's key tiles.  dQ_i = (1 / l_i) sum_j e_ij
  // (dP_ij - D_i) K_j is linear in the unnormalised weights e_ij, so it is
  // accumulated with the forward's online softmax: weights against a running
  // reference m, raised lazily (acc and l rescaled), divided by l at the end,
  // where lse = m c + log2 l also falls out for the dK/dV kernel.
  RowRegs<C> rk, rv;  // K and V rows of the next tile
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m = kNegInf, l = 0.f;
  load_rows<T, C>(rk, kbase, 0, a.Nk, tid, a.kv_rowb);
  load_rows<T, C>(rv, vbase, 0, a.Nk, tid, a.kv_rowb);
  store_rows<T, C>(rk, Krow(0), tid);
  store_rows<T, C>(rv, Vrow(0), tid);
  store_rows_t<T, C>(rk, Kt(0), tid);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt % NBUF;
    if (kt + 1 < ntiles) {
      load_rows<T, C>(rk, kbase, (kt + 1) * C::BC, a.Nk, tid, a.kv_rowb);
      load_rows<T, C>(rv, vbase, (kt + 1) * C::BC, a.Nk, tid, a.kv_rowb);
    }
    f32x16 s[C::KB], dp[C::KB];
    qk_tile<T, C>(s, qf, Krow(cur), j, h2);    // S^T = K Q^T
    qk_tile<T, C>(dp, dof, Vrow(cur), j, h2);  // dP^T = V dO^T
    const int key0 = kt * C::BC;
    if (key0 + C::BC > full_lim) mask_tile<C>(s, key0, lim, h2);
    // key 0 is visible to every row, so the first tile raises m in every lane
    const float mt = tile_rowmax<C>(s);
    if (__any(mt > m + a.thr)) raise_reference<C>(m, l, acc, mt, c);
    const float mc = m * c;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(s[kb][r], c, -mc));  // masked: 0
        l += e;
        s[kb][r] = e * (dp[kb][r] - Dv);
      }
    typename C::Frag dsf[C::KB][C::PF];
    to_frag<C>(s, dsf);
    pv_tile<T, C>(acc, dsf, Kt(cur), j, h2);  // dQ^T += K^T dS^T (unnormalised)
    if (kt + 1 < ntiles) {
      // with two buffers the other one was last read in step kt - 1, before
      // the barrier that ended it; with one, wait for every wave here
      if (NBUF == 1) __syncthreads();
      const int nxt = (cur + 1) % NBUF;
      store_rows<T, C>(rk, Krow(nxt), tid);
      store_rows<T, C>(rv, Vrow(nxt), tid);
      store_rows_t<T, C>(rk, Kt(nxt), tid);
    }
    __syncthreads();
  }
  const float lsum = halves_sum(l);
  const float lse = m * c + log2f(lsum);

  if (col.valid) {
    store_out_row<T, C>(reinterpret_cast<T*>(ba.dq) + col.row_off, acc, ba.scale / lsum, h2);
    if (h2 == 0) {
      const size_t row = col.row_off / C::D;  // contiguous rows
      ba.lse[row] = lse;
      ba.dd[row] = Dv;
    }
  }
}

// grid (ceil(Nk / (32 NW)) * qsplit, Hkv, B), C::NT threads: wave
// w owns keys k0 + 32 w .. k0 + 32 w + 31 of K/V head (b, hkv), over part
// `part` of the block's query steps; it writes fp32 partial dK (scaled) and
// dV to the part's records.  With two LDS buffers the staged query tiles
// alternate: tile st + 1 is written while tile st is used, so the LDS
// writes (and their wait for the tile's global loads) leave the critical
// path and one barrier per step remains.
template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) bwd_dkdv_kernel(BwdArgs ba) {
  const PrefillArgs& a = ba.f;
  constexpr int NBUF = bwd_buffers<C>();
  __shared__ __attribute__((aligned(16))) char smem[2 * NBUF * C::STAGE_BYTES];
  // buffer sg: Q row-major + dO transposed, then dO row-major + Q transposed
  auto KsA = [&](int sg) { return reinterpret_cast<T*>(smem + 2 * sg * C::STAGE_BYTES); };
  auto VsA = [&](int sg) { return KsA(sg) + C::K_ELEMS; };
  auto KsB = [&](int sg) { return reinterpret_cast<T*>(smem + (2 * sg + 1) * C::STAGE_BYTES); };
  auto VsB = [&](int sg) { return KsB(sg) + C::K_ELEMS; };
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // a batch's blocks in (key block, part, K/V head) order, heads fastest:
  // the heaviest key blocks of a causal launch, of every head, come first,
  // and consecutive blocks (on different XCDs) take different heads
  const int lin = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int hkv = lin % a.Hkv;
  const int part = (lin / a.Hkv) % ba.qsplit;
  const int k0 = (lin / a.Hkv / ba.qsplit) * 32 * C::NW;
  const int b = blockIdx.z;
  const int key = k0 + 32 * w + j;
  const bool kvalid = key < a.Nk;
  const size_t key_row = ((size_t)(b * a.Hkv + hkv) * a.Nk + (kvalid ? key : 0)) * C::D;
  typename C::Frag kf[C::QF], vf[C::QF];
  load_q_frag<T, C>(kf, reinterpret_cast<const T*>(a.k) + key_row, kvalid, false, h2);
  load_q_frag<T, C>(vf, reinterpret_cast<const T*>(a.v) + key_row, kvalid, false, h2);

  // query tiles: every head of the group, positions from the first tile
  // whose rows can see a key of this workgroup
  const int first = CAUSAL ? max(0, k0 - a.q_offset) / C::BC : 0;
  const int nqt = (a.Nq + C::BC - 1) / C::BC - first;  // >= 1 for launched blocks
  const int nall = a.g * nqt;  // query steps of the key block
  const int per_part = (nall + ba.qsplit - 1) / ba.qsplit;
  const int st0 = min(nall, part * per_part);
  const int nsteps = max(0, min(nall, st0 + per_part) - st0);  // this part's steps
  const float c = a.c;
  const int rowb = C::D * C::ESZ;

  f32x16 acc_dk[C::DB], acc_dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    acc_dk[db] = f32x16{};
    acc_dv[db] = f32x16{};
  }
  RowRegs<C> rq, rdo;  // Q and dO rows of the next tile
  // row statistics of a tile, per accumulator register: register r of
  // block kb is query row 32 kb + key_of_reg(r, h2), i.e. runs of 8
  // consecutive rows -- two 16-byte loads per run, through a resource over
  // the whole statistics area (reads past its end return 0; rows past Nq
  // are excluded below whatever they read)
  const auto stats = buffer_rsrc(
      ba.lse, __builtin_amdgcn_readfirstlane((uint32_t)(2ull * a.B * a.Hq * a.Nq * 4)));
  const uint32_t dd_off = (uint32_t)((size_t)a.B * a.Hq * a.Nq * 4);
  float4 lse4[C::KB][4], dd4[C::KB][4];
  // step st of this part is step st0 + st of the key block
  auto tile_head = [&](int st) { return hkv * a.g + (st0 + st) / nqt; };
  auto tile_i0 = [&](int st) { return (first + (st0 + st) % nqt) * C::BC; };
  auto issue = [&](int st) {
    const size_t hoff = (size_t)(b * a.Hq + tile_head(st)) * a.Nq * C::D;
    const T* qbase = uniform_ptr(reinterpret_cast<const T*>(a.q) + hoff);
    const T* dobase = uniform_ptr(reinterpret_cast<const T*>(ba.dout) + hoff);
    load_rows<T, C>(rq, qbase, tile_i0(st), a.Nq, tid, rowb);
    load_rows<T, C>(rdo, dobase, tile_i0(st), a.Nq, tid, rowb);
    const uint32_t srow = (uint32_t)((size_t)(b * a.Hq + tile_head(st)) * a.Nq + tile_i0(st));
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // registers 4 q4 .. 4 q4 + 3: rows 16 (q4 / 2) + 8 h2 + 4 (q4 % 2) + 0..3
        const uint32_t off =
            4u * (srow + 32 * kb + 16 * (q4 / 2) + 8 * h2 + 4 * (q4 % 2));
        lse4[kb][q4] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(stats, (int)off, 0, 0));
        dd4[kb][q4] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(stats, (int)(off + dd_off), 0, 0));
      }
  };
  if (nsteps > 0) {
    issue(0);
    store_rows<T, C>(rq, KsA(0), tid);
    store_rows_t<T, C>(rdo, VsA(0), tid);
    store_rows<T, C>(rdo, KsB(0), tid);
    store_rows_t<T, C>(rq, VsB(0), tid);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    const int cur = st % NBUF;
    const int i0 = tile_i0(st);
    float lse_r[C::KB][16], dd_r[C::KB][16];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        lse_r[kb][4 * q4] = lse4[kb][q4].x;
        lse_r[kb][4 * q4 + 1] = lse4[kb][q4].y;
        lse_r[kb][4 * q4 + 2] = lse4[kb][q4].z;
        lse_r[kb][4 * q4 + 3] = lse4[kb][q4].w;
        dd_r[kb][4 * q4] = dd4[kb][q4].x;
        dd_r[kb][4 * q4 + 1] = dd4[kb][q4].y;
        dd_r[kb][4 * q4 + 2] = dd4[kb][q4].z;
        dd_r[kb][4 * q4 + 3] = dd4[kb][q4].w;
      }
    if (st + 1 < nsteps) issue(st + 1);
    f32x16 s[C::KB], dp[C::KB];
    qk_tile<T, C>(s, kf, KsA(cur), j, h2);   // S = Q K^T
    qk_tile<T, C>(dp, vf, KsB(cur), j, h2);  // dP = dO V^T
    // every row of the tile exists and sees every key of this wave: no
    // per-element test (wave-uniform)
    const bool whole = i0 + C::BC <= a.Nq && (!CAUSAL || k0 + 32 * w + 31 <= a.q_offset + i0);
    if (whole) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse_r[kb][r]));
          s[kb][r] = p;
          dp[kb][r] = p * (dp[kb][r] - dd_r[kb][r]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // query row of accumulator register r; rows past Nq (zero Q and
          // dO) and, when causal, rows that cannot see this key weigh 0
          const int qi = i0 + 32 * kb + key_of_reg(r, h2);
          const bool vis = qi < a.Nq && (!CAUSAL || key <= a.q_offset + qi);
          const float p = vis ? fast_exp2(__builtin_fmaf(s[kb][r], c, -lse_r[kb][r])) : 0.f;
          s[kb][r] = p;
          dp[kb][r] = p * (dp[kb][r] - dd_r[kb][r]);
        }
    }
    typename C::Frag pf[C::KB][C::PF], dsf[C::KB][C::PF];
    to_frag<C>(s, pf);
    to_frag<C>(dp, dsf);
    pv_tile<T, C>(acc_dv, pf, VsA(cur), j, h2);   // dV^T += dO^T P
    pv_tile<T, C>(acc_dk, dsf, VsB(cur), j, h2);  // dK^T += Q^T dS
    if (st + 1 < nsteps) {
      // with two buffers the other one was last read in step st - 1, before
      // the barrier that ended it; with one, wait for every wave here
      if (NBUF == 1) __syncthreads();
      const int nxt = (cur + 1) % NBUF;
      store_rows<T, C>(rq, KsA(nxt), tid);
      store_rows_t<T, C>(rdo, VsA(nxt), tid);
      store_rows<T, C>(rdo, KsB(nxt), tid);
      store_rows_t<T, C>(rq, VsB(nxt), tid);
    }
    __syncthreads();
  }

  if (kvalid && ba.qsplit == 1) {  // one part: the result itself
    store_out_row<T, C>(reinterpret_cast<T*>(ba.dk) + key_row, acc_dk, ba.scale, h2);
    store_out_row<T, C>(reinterpret_cast<T*>(ba.dv) + key_row, acc_dv, 1.0f, h2);
  } else if (kvalid) {
    // records [part][dK, dV][b][hkv][key][D], fp32; this lane holds
    // d = 32 db + 8 q4 + 4 h2 + 0..3
    const size_t rows = (size_t)a.B * a.Hkv * a.Nk;
    const size_t krow = (size_t)(b * a.Hkv + hkv) * a.Nk + key;
    float* pk = ba.part + ((size_t)(2 * part) * rows + krow) * C::D;
    float* pv = ba.part + ((size_t)(2 * part + 1) * rows + krow) * C::D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * h2;
        *reinterpret_cast<float4*>(pk + d0) =
            float4{acc_dk[db][4 * q4] * ba.scale, acc_dk[db][4 * q4 + 1] * ba.scale,
                   acc_dk[db][4 * q4 + 2] * ba.scale, acc_dk[db][4 * q4 + 3] * ba.scale};
        *reinterpret_cast<float4*>(pv + d0) = float4{acc_dv[db][4 * q4], acc_dv[db][4 * q4 + 1],
                                                     acc_dv[db][4 * q4 + 2], acc_dv[db][4 * q4 + 3]};
      }
  }
}

typedef float acc4 __attribute__((ext_vector_type(4)));

// bf16 dK/dV on the 16x16x32 MFMA: 16 keys per wave, four waves (64 keys)
// per workgroup, the same grid, query parts and records as bwd_dkdv_kernel.
// Half the keys per wave halves the accumulators and the K/V fragments, so
// two waves fit on each SIMD (the 32-key kernel holds one).  In one step a
// wave forms, for a staged 32-query tile (C: its LDS layout, the 4-wave
// staging of bwd_dkdv_kernel),
//   S = Q K^T and dP = dO V^T: two 16-query blocks, A = Q (or dO) rows from
//   LDS, B = the wave's K (or V) fragment in registers; MFMA row m of block
//   qb reads query 8 (m / 4) + 4 qb + m % 4, so that lane (n, G) ends up
//   with queries 8 G .. 8 G + 7 of its key n -- exactly the B operand the
//   next products take (the row permutation of the decode part kernel);
//   dV^T += dO^T P and dK^T += Q^T dS: D / 16 blocks of 16 head dims,
//   A = dO^T (or Q^T) from the transposed LDS copy, B = P (or dS) from
//   registers.
template <class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkdv16_kernel(BwdArgs ba) {
  using T = uint16_t;
  static_assert(!C::F32 && C::BC == 32 && C::NW == 4, "bf16, 32-query tiles, 4 waves");
  constexpr int D = C::D;
  constexpr int DT = D / 32;  // 32-deep steps of the score MFMAs
  constexpr int DB = D / 16;  // 16-row blocks of dK^T and dV^T
  const PrefillArgs& a = ba.f;
  constexpr int NBUF = bwd_buffers<C>();
  __shared__ __attribute__((aligned(16))) char smem[2 * NBUF * C::STAGE_BYTES];
  // buffer sg: Q row-major + dO transposed, then dO row-major + Q transposed
  auto KsA = [&](int sg) { return reinterpret_cast<T*>(smem + 2 * sg * C::STAGE_BYTES); };
  auto VsA = [&](int sg) { return KsA(sg) + C::K_ELEMS; };
  auto KsB = [&](int sg) { return reinterpret_cast<T*>(smem + (2 * sg + 1) * C::STAGE_BYTES); };
  auto VsB = [&](int sg) { return KsB(sg) + C::K_ELEMS; };
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;  // the lane's key within the wave's 16
  const int G = lane >> 4;  // the lane's group: queries 8 G .. 8 G + 7 of a tile

  // a batch's blocks in (key block, part, K/V head) order, heads fastest:
  // the heaviest key blocks of a causal launch, of every head, come first,
  // and consecutive blocks (on different XCDs) take different heads
  const int lin = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int hkv = lin % a.Hkv;
  const int part = (lin / a.Hkv) % ba.qsplit;
  const int k0 = (lin / a.Hkv / ba.qsplit) * 64;
  const int b = blockIdx.z;
  const int key = k0 + 16 * w + n;
  const bool kvalid = key < a.Nk;
  const size_t key_row = ((size_t)(b * a.Hkv + hkv) * a.Nk + (kvalid ? key : 0)) * D;
  bf16x8 kf[DT], vf[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 kw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.k) + key_row + 32 * t + 8 * G);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.v) + key_row + 32 * t + 8 * G);
    kf[t] = __builtin_bit_cast(bf16x8, kvalid ? kw : zero);
    vf[t] = __builtin_bit_cast(bf16x8, kvalid ? vw : zero);
  }

  const int first = CAUSAL ? max(0, k0 - a.q_offset) / C::BC : 0;
  const int nqt = (a.Nq + C::BC - 1) / C::BC - first;  // >= 1 for launched blocks
  const int nall = a.g * nqt;
  const int per_part = (nall + ba.qsplit - 1) / ba.qsplit;
  const int st0 = min(nall, part * per_part);
  const int nsteps = max(0, min(nall, st0 + per_part) - st0);
  const float c = a.c;
  const int rowb = D * C::ESZ;

  acc4 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc_dk[db] = acc4{0.f, 0.f, 0.f, 0.f};
    acc_dv[db] = acc4{0.f, 0.f, 0.f, 0.f};
  }
  RowRegs<C> rq, rdo;  // Q and dO rows of the next tile
  // row statistics of the lane's 8 queries, through a resource over the
  // whole statistics area (rows past Nq read the next head's values or
  // zeros; they are excluded below whatever they read)
  const auto stats = buffer_rsrc(
      ba.lse, __builtin_amdgcn_readfirstlane((uint32_t)(2ull * a.B * a.Hq * a.Nq * 4)));
  const uint32_t dd_off = (uint32_t)((size_t)a.B * a.Hq * a.Nq * 4);
  float4 lse4[2], dd4[2];
  auto tile_head = [&](int st) { return hkv * a.g + (st0 + st) / nqt; };
  auto tile_i0 = [&](int st) { return (first + (st0 + st) % nqt) * C::BC; };
  auto issue = [&](int st) {
    const size_t hoff = (size_t)(b * a.Hq + tile_head(st)) * a.Nq * D;
    const T* qbase = uniform_ptr(reinterpret_cast<const T*>(a.q) + hoff);
    const T* dobase = uniform_ptr(reinterpret_cast<const T*>(ba.dout) + hoff);
    load_rows<T, C>(rq, qbase, tile_i0(st), a.Nq, tid, rowb);
    load_rows<T, C>(rdo, dobase, tile_i0(st), a.Nq, tid, rowb);
    const uint32_t off =
        4u * (uint32_t)((size_t)(b * a.Hq + tile_head(st)) * a.Nq + tile_i0(st) + 8 * G);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lse4[h] = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(stats, (int)(off + 16 * h), 0, 0));
      dd4[h] = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(stats, (int)(off + 16 * h + dd_off), 0, 0));
    }
  };
  auto stage = [&](int sg) {
    store_rows<T, C>(rq, KsA(sg), tid);
    store_rows_t<T, C>(rdo, VsA(sg), tid);
    store_rows<T, C>(rdo, KsB(sg), tid);
    store_rows_t<T, C>(rq, VsB(sg), tid);
  };
  if (nsteps > 0) {
    issue(0);
    stage(0);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    const int cur = st % NBUF;
    const int i0 = tile_i0(st);
    float lse_r[8], dd_r[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lse_r[4 * h] = lse4[h].x;
      lse_r[4 * h + 1] = lse4[h].y;
      lse_r[4 * h + 2] = lse4[h].z;
      lse_r[4 * h + 3] = lse4[h].w;
      dd_r[4 * h] = dd4[h].x;
      dd_r[4 * h + 1] = dd4[h].y;
      dd_r[4 * h + 2] = dd4[h].z;
      dd_r[4 * h + 3] = dd4[h].w;
    }
    if (st + 1 < nsteps) issue(st + 1);
    acc4 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = 8 * (n >> 2) + 4 * qb + (n & 3);
      const T* qr = KsA(cur) + row * C::KSTR + 8 * G;
      const T* dr = KsB(cur) + row * C::KSTR + 8 * G;
      bf16x8 qa[DT], da[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        qa[t] = *reinterpret_cast<const bf16x8*>(qr + 32 * t);
        da[t] = *reinterpret_cast<const bf16x8*>(dr + 32 * t);
      }
      acc4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], kf[t], x, 0, 0, 0);  // S = Q K^T
        y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[t], vf[t], y, 0, 0, 0);  // dP = dO V^T
      }
      s[qb] = x;
      dp[qb] = y;
    }
    // element i of block qb: query 8 G + 4 qb + i, key n of the wave
    const bool whole = i0 + C::BC <= a.Nq && (!CAUSAL || k0 + 16 * w + 15 <= a.q_offset + i0);
    float p[8], ds[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = s[e >> 2][e & 3];
      float pv = fast_exp2(__builtin_fmaf(sv, c, -lse_r[e]));
      if (!whole) {
        // rows past Nq (zero Q and dO) and, when causal, rows that cannot
        // see this key weigh 0
        const int qi = i0 + 8 * G + e;
        const bool vis = qi < a.Nq && (!CAUSAL || key <= a.q_offset + qi);
        pv = vis ? pv : 0.f;
      }
      p[e] = pv;
      ds[e] = pv * (dp[e >> 2][e & 3] - dd_r[e]);
    }
    u32x4 pw, dw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pw[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
      dw[e] = pack_bf16(ds[2 * e], ds[2 * e + 1]);
    }
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    const bf16x8 dsf = __builtin_bit_cast(bf16x8, dw);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 ao = *reinterpret_cast<const bf16x8*>(VsA(cur) + (16 * db + n) * C::VSTR + 8 * G);
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(VsB(cur) + (16 * db + n) * C::VSTR + 8 * G);
      acc_dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, pf, acc_dv[db], 0, 0, 0);   // dV^T += dO^T P
      acc_dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, dsf, acc_dk[db], 0, 0, 0);  // dK^T += Q^T dS
    }
    if (st + 1 < nsteps) {
      // with two buffers the other one was last read in step st - 1, before
      // the barrier that ended it; with one, wait for every wave here
      if (NBUF == 1) __syncthreads();
      stage((cur + 1) % NBUF);
    }
    __syncthreads();
  }

  // the lane holds head dims 16 db + 4 G .. + 3 of key n
  if (kvalid && ba.qsplit == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = 16 * db + 4 * G;
      const acc4 k4 = acc_dk[db] * ba.scale;
      const acc4 v4 = acc_dv[db];
      *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(ba.dk) + key_row + d0) =
          u32x2{pack_bf16(k4[0], k4[1]), pack_bf16(k4[2], k4[3])};
      *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(ba.dv) + key_row + d0) =
          u32x2{pack_bf16(v4[0], v4[1]), pack_bf16(v4[2], v4[3])};
    }
  } else if (kvalid) {
    // records [part][dK, dV][b][hkv][key][D], fp32
    const size_t rows = (size_t)a.B * a.Hkv * a.Nk;
    const size_t krow = (size_t)(b * a.Hkv + hkv) * a.Nk + key;
    float* pk = ba.part + ((size_t)(2 * part) * rows + krow) * D;
    float* pv = ba.part + ((size_t)(2 * part + 1) * rows + krow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = 16 * db + 4 * G;
      const acc4 k4 = acc_dk[db] * ba.scale;
      *reinterpret_cast<float4*>(pk + d0) = float4{k4[0], k4[1], k4[2], k4[3]};
      *reinterpret_cast<float4*>(pv + d0) =
          float4{acc_dv[db][0], acc_dv[db][1], acc_dv[db][2], acc_dv[db][3]};
    }
  }
}

// dK, dV = the sum of the query parts' records, in part order, rounded
// once to the output type.  One thread per 4 consecutive elements of
// dK or dV; n4 = 2 * B * Hkv * Nk * D / 4.
template <typename T>
__global__ void __launch_bounds__(256) bwd_merge_kernel(BwdArgs ba, long long n4) {
  const long long half4 = n4 / 2;  // float4s of dK (then as many of dV)
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const bool is_v = i >= half4;
    const long long e4 = is_v ? i - half4 : i;
    const float4* src = reinterpret_cast<const float4*>(ba.part) + (is_v ? half4 : 0) + e4;
    float4 acc = src[0];
    for (int p = 1; p < ba.qsplit; ++p) {
      const float4 x = src[(long long)p * n4];
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    T* dst = reinterpret_cast<T*>(is_v ? ba.dv : ba.dk) + 4 * e4;
    if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<float4*>(dst) = acc;
    } else {
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16(acc.x, acc.y), pack_bf16(acc.z, acc.w)};
    }
  }
}

}  // namespace gqa
