// prefill_kernel.hpp -- GQA forward (prefill and chunked prefill).
//
// Work unit = (batch b, K/V head hkv, head block hb, position block qb): the
// Gu query heads hb*Gu .. hb*Gu+Gu-1 of the group that shares K/V head hkv
// (head mapping hkv = h / g, BootstrapAI evolution log, "Kernel 9 -- GQA"),
// stacked over R consecutive query positions, Gu*R <= 32*NW columns.  Column
// m of the unit is head r = m / R at position p = m % R, so every K/V tile a
// workgroup stages in LDS is read from HBM once and serves all Gu heads: the
// "one K/V tile shared by many query rows" idea of the same log's
// cooperative-loading kernel ("Kernel 3"), widened from query rows to the
// whole head group.  The units of one (b, hkv, hb) form a slice.
//
// Two schedules share the per-unit code:
//
// * prefill_kernel, for launches with many units, is persistent ("Kernel 8 --
//   persistent kernel" of the same log): the grid holds as many workgroups
//   as fit on the device at once and each repeatedly takes the next unit
//   from a device counter with one atomic add.  The units are split into
//   kNumQueues queues by K/V group (b*Hkv + hkv) modulo kNumQueues, one per
//   XCD: workgroups are dispatched to the XCDs round-robin by block index, so
//   a workgroup first drains the queue of its own XCD and the K/V tiles of a
//   group stay in that XCD's L2; once its queue is empty it looks at all
//   queues at once and steals.  Within a queue units are numbered heaviest
//   first for causal attention (the last position blocks see the most keys),
//   which makes the first-come order a longest-job-first schedule.  The last
//   workgroup to leave resets the counters for the next launch.
//
// * prefill_balanced_kernel, for launches with about as many units as
//   resident workgroups or fewer, where whole units cannot be balanced: each
//   slice's key tiles, taken unit after unit, form one sequence that is cut
//   into Pp equal chunks, one per workgroup.  A chunk covers the end of one
//   unit, whole units and the start of another; a unit cut by a chunk
//   boundary leaves partial softmax states (m, l, unnormalised O) that
//   prefill_merge_kernel combines.  For causal attention the units are
//   ordered heavy, light, heavy, light (qb = NQB-1, 0, NQB-2, 1, ...), so
//   that the chunk boundaries fall mostly between units.
//
// Per unit the key tiles stream through a two-stage LDS ring fed from two
// register staging sets, so each tile's global loads are issued two tiles
// before they are needed.  Causal masking runs only on tiles that cross the
// diagonal (or the ragged end of the keys); tiles above the diagonal of the
// whole unit are never loaded.
#pragma once

#include "attn_tile.hpp"

namespace gqa {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, Hq, Hkv, Nq, Nk;
  // element strides (batch, head, token; d is contiguous): one set for Q and
  // O, one for K and V
  long long q_sb, q_sh, q_sn;
  long long kv_sb, kv_sh;
  int kv_rowb;  // K/V token stride in bytes
  int g;    // Hq / Hkv
  int Gu;   // query heads per unit
  int R;    // query positions per unit
  int HB;   // head blocks per K/V head, ceil(g / Gu)
  int NQB;  // position blocks, ceil(Nq / R)
  int T;    // units, B * Hkv * HB * NQB
  int q_offset;
  float c;    // |scale| * log2(e)
  float thr;  // kRescaleSlack / c: how far a tile max may exceed the reference
  int negate_q;
  // balanced schedule: slices, chunks per slice, key tiles per slice, and
  // two partial records per workgroup (first and last segment)
  int nsl;
  int Pp;
  int Ws;
  float* ws;
  int zero;  // always 0 (the probe's atomic add, kept a read-modify-write)
  int* ctr;  // counter i at ctr[i * kCounterStride]: next item of queue i < kNumQueues,
             // workgroups finished for i = kNumQueues
  // packed varlen batches: sequence b owns query rows [cu_q[b], cu_q[b+1])
  // and key rows [cu_k[b], cu_k[b+1]) of token-major tensors (NULL otherwise)
  const int32_t* cu_q;
  const int32_t* cu_k;
};

constexpr int kNumQueues = 8;  // XCDs of an MI355X
// Scheduler counters sit 256 bytes apart, each in a cache line (and memory
// channel) of its own, so that the atomics of different queues do not queue
// up behind one another.
constexpr int kCounterStride = 64;
// Pieces of one unit under the balanced schedule, at most.
constexpr int kMaxPiecesDev = 16;

// Items in queue q: the K/V groups q, q + kNumQueues, ... below nkv.
__device__ __forceinline__ int queue_units(int q, int nkv, int per_group) {
  return nkv > q ? ((nkv - q + kNumQueues - 1) / kNumQueues) * per_group : 0;
}

// Floats of one partial record (one key-range part of one unit): for each of
// the NW waves, its DB*16 accumulator registers as DB*4 rows of 64 lanes x 4
// floats (one coalesced 1 KiB row per 16-byte access), then the running
// reference m and per-lane sum l as 64 lane pairs.
template <class C>
constexpr int wave_record_floats() {
  return (C::DB * 16 + 2) * 64;
}
template <class C>
constexpr int part_floats() {
  return C::NW * wave_record_floats<C>();
}

// Key tiles of the units of position block qb.
template <class C, bool CAUSAL>
__device__ __forceinline__ int unit_tiles(const PrefillArgs& a, int qb) {
  const int i_hi = min(a.Nq, (qb + 1) * a.R) - 1;
  const int kend = CAUSAL ? min(a.Nk, a.q_offset + i_hi + 1) : a.Nk;
  return (kend + C::BC - 1) / C::BC;
}

// Position pos of a slice's unit sequence -> position block.  Causal:
// heavy and light units alternate (NQB-1, 0, NQB-2, 1, ...).
template <bool CAUSAL>
__device__ __forceinline__ int seq_qb(int pos, int NQB) {
  if (!CAUSAL) return pos;
  return (pos & 1) ? (pos >> 1) : NQB - 1 - (pos >> 1);
}

// First tile of chunk c of a slice (chunk c covers [bound(c), bound(c+1))).
__device__ __forceinline__ int chunk_bound(const PrefillArgs& a, int c) {
  return (int)((long long)c * a.Ws / a.Pp);
}

// Locates tile X (0 <= X < Ws) of the slice sequence: the sequence position
// holding it and the number of tiles before that position.  Called by a
// whole wave; every lane returns the same result.  Each lane sums the tile
// counts of a contiguous run of positions, a wave prefix sum finds the run
// holding X, and a short walk inside it finds the position.
template <class C, bool CAUSAL>
__device__ __forceinline__ void locate_tile(const PrefillArgs& a, int X, int lane, int& pos_out,
                                            int& pre_out) {
  const int E = (a.NQB + 63) / 64;
  const int p0 = min(a.NQB, lane * E);
  const int p1 = min(a.NQB, p0 + E);
  int sum = 0;
  for (int p = p0; p < p1; ++p) sum += unit_tiles<C, CAUSAL>(a, seq_qb<CAUSAL>(p, a.NQB));
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - sum;
  const unsigned long long hit = __ballot(excl <= X && X < incl);
  const int L = hit ? __ffsll((long long)hit) - 1 : 63;
  int pre = __shfl(excl, L);
  int pos = __shfl(p0, L);
  for (;;) {
    const int n = unit_tiles<C, CAUSAL>(a, seq_qb<CAUSAL>(pos, a.NQB));
    if (pre + n > X || pos + 1 >= a.NQB) break;
    pre += n;
    ++pos;
  }
  pos_out = __builtin_amdgcn_readfirstlane(pos);  // the same in every lane
  pre_out = __builtin_amdgcn_readfirstlane(pre);
}

// Partial record `slot` (0: first segment, 1: last segment) of workgroup g
// of the balanced schedule.
template <class C>
__device__ __forceinline__ float* part_record(const PrefillArgs& a, int g, int slot) {
  return a.ws + ((size_t)g * 2 + slot) * part_floats<C>();
}

// The query column a lane owns: column m = 32 w + j of the unit is head
// r = m / R of the head block at position p = m % R.
struct Column {
  bool valid;
  int i;           // query row
  size_t row_off;  // element offset of the row in Q and O
};

template <class C>
__device__ __forceinline__ Column lane_column(const PrefillArgs& a, int b, int hkv, int hb, int qb,
                                              int w, int j) {
  const int m = 32 * w + j;
  const int r = m / a.R;
  const int p = m - r * a.R;
  const int hig = hb * a.Gu + r;  // head within the group
  Column c;
  c.i = qb * a.R + p;
  c.valid = (r < a.Gu) && (hig < a.g) && (c.i < a.Nq);
  const int h = hkv * a.g + hig;
  c.row_off = c.valid ? (size_t)(b * a.q_sb + h * a.q_sh + c.i * a.q_sn) : 0;
  return c;
}

// What a segment needs before its first step, in registers: the Q fragment
// and the loads of its first two tiles.  Issuing them early (seg_begin) and
// running the segment later (seg_run) lets a caller hide their latency
// behind other work.
template <class C>
struct SegIn {
  typename C::Frag qf[C::QF];
  TileRegs<C> ra, rb;
};

// The tiles of a segment: [tile0, tile0 + ntiles) walked from rotation rot;
// positions past the end repeat the last one.  An empty range (possible for
// a paired half) always yields tile0, which must be a valid tile.
struct SegTiles {
  int tile0, ntiles, rot;
  __device__ __forceinline__ int at(int pos) const {
    if (ntiles == 0) return tile0;
    const int x = (pos < ntiles ? pos : ntiles - 1) + rot;
    return tile0 + (x >= ntiles ? x - ntiles : x);
  }
};

template <typename T, class C>
__device__ __forceinline__ void kv_bases(const PrefillArgs& a, int b, int hkv, const T*& kbase,
                                         const T*& vbase) {
  const size_t kv_off = (size_t)(b * a.kv_sb + hkv * a.kv_sh);
  kbase = uniform_ptr(reinterpret_cast<const T*>(a.k) + kv_off);
  vbase = uniform_ptr(reinterpret_cast<const T*>(a.v) + kv_off);
}

// K1 false: tile 1's K rows are not loaded (seg_run_direct loads them
// straight into LDS).
template <typename T, class C, bool K1 = true>
__device__ __forceinline__ void seg_begin(const PrefillArgs& a, SegIn<C>& in, int b, int hkv,
                                          const SegTiles& st, const Column& col) {
  const int tid = threadIdx.x % C::NT;  // index within the loading group
  const int h2 = (tid & 63) >> 5;
  const T* kbase;
  const T* vbase;
  kv_bases<T, C>(a, b, hkv, kbase, vbase);
  load_q_frag<T, C>(in.qf, reinterpret_cast<const T*>(a.q) + col.row_off, col.valid,
                    a.negate_q != 0, h2);
  load_tile<T, C>(in.ra, kbase, vbase, st.at(0) * C::BC, a.Nk, tid, a.kv_rowb);
  load_tile<T, C, K1>(in.rb, kbase, vbase, st.at(1) * C::BC, a.Nk, tid, a.kv_rowb);
}

// Runs key tiles st of unit (b, hkv, ., qb) for the lane's column col, from
// the registers seg_begin filled, and leaves the running state (reference
// m, per-lane sum l and unnormalised O) in mrun, lrun, acc.  All threads of
// the workgroup call it together; it ends on a barrier, so the LDS ring is
// free on return.
//
// PAIRED: two groups of NW waves (one per half of the workgroup) run the
// function together on their own LDS rings, each over its own tile range;
// both loop `steps` times (the longer range) so that they meet at every
// barrier, and a group whose range is shorter skips the compute of its last
// steps.
//
// Two LDS stages and two register staging sets: the global loads of tile
// t+2 are issued at the start of tile t and written to LDS at the end of
// tile t+1, so two tiles of compute cover their latency.  The loop is
// unrolled by two so each staging set is a named register set, and the
// loads and stores are unconditional (indices clamped to the last tile) so
// the compiler's wait before each LDS store counts exactly the newer loads
// still in flight.
//
// The tiles are walked from a caller-chosen rotation, so the many
// workgroups that share a K/V head do not all request the same tile at the
// same moment.  The order of tiles does not change the result in exact
// arithmetic (masking is per key, and a lane whose first tiles are all
// masked keeps an empty state until a visible key comes).
template <typename T, class C, bool CAUSAL, bool PAIRED = false>
__device__ __forceinline__ void seg_run(const PrefillArgs& a, char* smem, SegIn<C>& in, int b,
                                        int hkv, int qb, const SegTiles& st, const Column& col,
                                        float& mrun, float& lrun, f32x16 (&acc)[C::DB],
                                        int steps) {
  const int tid = threadIdx.x % C::NT;  // index within the loading group
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;
  auto stK = [&](int sg) { return reinterpret_cast<T*>(smem + sg * C::STAGE_BYTES); };
  auto stV = [&](int sg) { return stK(sg) + C::K_ELEMS; };
  const T* kbase;
  const T* vbase;
  kv_bases<T, C>(a, b, hkv, kbase, vbase);

  // keys below full_lim are visible to every column of the unit; lim is the
  // last key this lane's query may see
  const int full_lim = CAUSAL ? min(a.Nk, a.q_offset + qb * a.R + 1) : a.Nk;
  const int lim = (CAUSAL && col.valid) ? min(a.q_offset + col.i, a.Nk - 1) : a.Nk - 1;

  mrun = kNegInf;
  lrun = 0.f;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  if (!PAIRED) steps = st.ntiles;
  store_tile<T, C>(in.ra, stK(0), stV(0), tid);
  __syncthreads();

  auto step = [&](TileRegs<C>& mine, TileRegs<C>& next, int kt) {
    const int cur = kt & 1;
    load_tile<T, C>(mine, kbase, vbase, st.at(kt + 2) * C::BC, a.Nk, tid, a.kv_rowb);
    if (!PAIRED || kt < st.ntiles) {
      f32x16 s[C::KB];
      qk_tile<T, C>(s, in.qf, stK(cur), j, h2);
      const int key0 = st.at(kt) * C::BC;
      if (key0 + C::BC > full_lim) mask_tile<C>(s, key0, lim, h2);
      softmax_pv_step<T, C>(s, mrun, lrun, acc, stV(cur), j, h2, a.c, a.thr);
    }
    store_tile<T, C>(next, stK(cur ^ 1), stV(cur ^ 1), tid);
    __syncthreads();
  };
  for (int kt = 0; kt < steps; kt += 2) {
    step(in.ra, in.rb, kt);
    if (kt + 1 < steps) step(in.rb, in.ra, kt + 1);
  }
}

// Whether the key-split schedules (pair and quad) stage K by direct
// global -> LDS loads instead of through registers: bf16, d = 128.
template <class C>
constexpr bool use_direct_k() {
  return direct_k_ok<C>() && C::D == 128;
}

// LDS ring of seg_run_direct: two K slots (direct-load layout), then two
// V^T stages.
template <class C>
constexpr int dk_ring_bytes() {
  return 2 * dk_slot_bytes<C>() + 2 * C::V_ELEMS * 2;
}

// s_waitcnt immediate: at most n vector-memory loads outstanding (the
// other counters unconstrained).
constexpr int waitcnt_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// seg_run with K staged by direct loads (the caller's
// seg_begin<T, C, false> leaves tile 1's K rows unloaded): tile t + 1's K
// rows go straight into K slot (t + 1) & 1 at the start of tile t
// (that slot was last read in tile t - 1, before the barrier that ended
// it), and each wave waits for them before the barrier that ends tile t,
// which then publishes them; V is staged as in seg_run (registers two tiles
// ahead, then the transposing stores).  On return every load has completed
// (the ring may be reused at once) and the workgroup has passed a barrier.
template <typename T, class C, bool CAUSAL>
__device__ __forceinline__ void seg_run_direct(const PrefillArgs& a, char* ring, SegIn<C>& in,
                                               int b, int hkv, int qb, const SegTiles& st,
                                               const Column& col, float& mrun, float& lrun,
                                               f32x16 (&acc)[C::DB], int steps) {
  static_assert(direct_k_ok<C>(), "direct K staging: bf16, d = 128 or 64");
  const int tid = threadIdx.x % C::NT;  // index within the loading group
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;
  auto kslot = [&](int sl) { return ring + sl * dk_slot_bytes<C>(); };
  auto vstage = [&](int sg) {
    return reinterpret_cast<T*>(ring + 2 * dk_slot_bytes<C>() + sg * C::V_ELEMS * 2);
  };
  const T* kbase;
  const T* vbase;
  kv_bases<T, C>(a, b, hkv, kbase, vbase);
  const KDirect<C> kd = k_direct_offsets<C>(tid, a.kv_rowb);
  // slot 0's K fragment addresses, computed once; the empty asm keeps them
  // in registers (left alone, the compiler re-adds the slot base to each
  // lane offset in every tile: eight more VALU instructions per tile)
  lds_cchar* kp[C::KB][C::QF];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int ks = 0; ks < C::QF; ++ks) {
      kp[kb][ks] = (lds_cchar*)(ring) +
                   dk_chunk_off<C>(32 * kb + k_row_perm(j), 2 * ks + h2);
      asm volatile("" : "+v"(kp[kb][ks]));
    }
  const int full_lim = CAUSAL ? min(a.Nk, a.q_offset + qb * a.R + 1) : a.Nk;
  const int lim = (CAUSAL && col.valid) ? min(a.q_offset + col.i, a.Nk - 1) : a.Nk - 1;

  mrun = kNegInf;
  lrun = 0.f;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  store_k_direct_layout<C>(in.ra, kslot(0), tid);
  store_tile<T, C, false>(in.ra, nullptr, vstage(0), tid);
  __syncthreads();

  // tile kt: K in slot kt & 1, V^T in stage kt & 1
  auto step = [&](TileRegs<C>& mine, TileRegs<C>& next, int kt, int cur) {
    k_direct<C>(kbase, st.at(kt + 1) * C::BC, a.Nk, kslot(cur ^ 1), tid, a.kv_rowb, kd.off);
    load_tile<T, C, false>(mine, kbase, vbase, st.at(kt + 2) * C::BC, a.Nk, tid, a.kv_rowb);
    if (kt < st.ntiles) {
      f32x16 s[C::KB];
      if (cur == 0)
        qk_tile_direct_at<C, 0>(s, in.qf, kp);
      else
        qk_tile_direct_at<C, 1>(s, in.qf, kp);
      const int key0 = st.at(kt) * C::BC;
      if (key0 + C::BC > full_lim) mask_tile<C>(s, key0, lim, h2);
      softmax_pv_step<T, C>(s, mrun, lrun, acc, vstage(cur), j, h2, a.c, a.thr);
    }
    store_tile<T, C, false>(next, nullptr, vstage(cur ^ 1), tid);
    // the K loads of tile kt + 1 (issued before this tile's V loads) are in
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::V_LOADS));
    __syncthreads();
  };
  for (int kt = 0; kt < steps; kt += 2) {
    step(in.ra, in.rb, kt, 0);
    if (kt + 1 < steps) step(in.rb, in.ra, kt + 1, 1);
  }
  // the last tile's K loads (of a tile past the range) may still be landing
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// seg_begin + seg_run (seg_run_direct for non-causal bf16 units at d = 128
// and 64) back to back.
template <typename T, class C, bool CAUSAL>
__device__ __forceinline__ void run_segment(const PrefillArgs& a, char* smem, int b, int hkv,
                                            int qb, int tile0, int ntiles, int rot,
                                            const Column& col, float& mrun, float& lrun,
                                            f32x16 (&acc)[C::DB]) {
  SegIn<C> in;
  const SegTiles st{tile0, ntiles, rot};
  // non-causal units are long (every key tile), so the direct K loads' one-tile
  // lead costs nothing at their start; causal ones keep the register path
  if constexpr (direct_k_ok<C>() && !CAUSAL) {
    static_assert(dk_ring_bytes<C>() <= 2 * C::STAGE_BYTES, "direct-K ring exceeds two stages");
    seg_begin<T, C, false>(a, in, b, hkv, st, col);
    seg_run_direct<T, C, CAUSAL>(a, smem, in, b, hkv, qb, st, col, mrun, lrun, acc, ntiles);
  } else {
    seg_begin<T, C>(a, in, b, hkv, st, col);
    seg_run<T, C, CAUSAL>(a, smem, in, b, hkv, qb, st, col, mrun, lrun, acc, ntiles);
  }
}

// Bytes of one wave's output staging area: its 32 rows of O with a
// 16-byte pad per row (which spreads the rows over the LDS banks).
template <class C>
constexpr int stage_out_bytes() {
  return 32 * (C::D * C::ESZ + 16);
}

// Normalises the lane's row of O by 1 / (the sum of its two half-waves) and
// stores the wave's 32 rows through `stg`, the wave's own staging area in
// LDS.  The rows go in as the MFMA layout holds them (4 elements per lane
// per block) and come out as 16-byte chunks of whole rows, so every store
// instruction writes complete rows: a direct store from the MFMA layout
// would write 8 bytes into each of 32 rows per instruction, and those
// partial-line writes are what an output costs most.
template <typename T, class C>
__device__ __forceinline__ void finish_rows(const PrefillArgs& a, char* stg, float lrun,
                                            const f32x16 (&acc)[C::DB], int b, int hkv, int hb,
                                            int qb, int w) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;
  constexpr int RB = C::D * C::ESZ + 16;  // staging row stride, bytes
  // a row that saw no key (possible only in a packed varlen batch whose
  // sequence has more queries than keys) has l = 0 and is zero
  const float lsum = halves_sum(lrun);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  char* row = stg + j * RB;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * h2;
      const float x0 = acc[db][4 * q4 + 0] * inv;
      const float x1 = acc[db][4 * q4 + 1] * inv;
      const float x2 = acc[db][4 * q4 + 2] * inv;
      const float x3 = acc[db][4 * q4 + 3] * inv;
      if constexpr (C::F32) {
        *reinterpret_cast<float4*>(row + d0 * 4) = float4{x0, x1, x2, x3};
      } else {
        *reinterpret_cast<u32x2*>(row + d0 * 2) = u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = C::D * C::ESZ / 16;  // 16-byte chunks per row
  constexpr int CPI = 64 / CPR;            // rows per store instruction
  const int ch = lane % CPR;
#pragma unroll
  for (int k = 0; k < 32 / CPI; ++k) {
    const int c = k * CPI + lane / CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + c * RB + ch * 16);
    const Column cc = lane_column<C>(a, b, hkv, hb, qb, w, c);
    if (cc.valid)
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.o) + cc.row_off * C::ESZ + ch * 16) = v;
  }
}

// Writes the wave's partial state to a record: the accumulator registers as
// rows of 64 lanes x 4 floats, then (m, l) per lane.
template <class C>
__device__ __forceinline__ void write_record(float* rec, float mrun, float lrun,
                                             const f32x16 (&acc)[C::DB], int w, int lane) {
  rec += w * wave_record_floats<C>();
  float4* rec4 = reinterpret_cast<float4*>(rec);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      rec4[(db * 4 + r4) * 64 + lane] = make_float4(acc[db][4 * r4], acc[db][4 * r4 + 1],
                                                    acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]);
  reinterpret_cast<float2*>(rec + C::DB * 16 * 64)[lane] = make_float2(mrun, lrun);
}

// Wave 0 of a persistent workgroup: the next item of the home queue; once
// that is empty, every queue is looked at at once (lane l reads queue
// home + l with an atomic add of zero) and an item is taken from the first
// that still has one.  Every failed take means the queue is empty for good,
// so this ends.  Returns t = -1 when every queue is empty; q is the queue
// of t.
__device__ __forceinline__ void take_unit(const PrefillArgs& a, int home, int nkv, int per_group,
                                          bool& home_empty, int lane, int& t_out, int& q_out) {
  int t = -1, q = home;
  if (!home_empty) {
    int cand = 0;
    if (lane == 0) cand = atomicAdd(a.ctr + home * kCounterStride, 1);
    cand = __shfl(cand, 0);
    if (cand < queue_units(home, nkv, per_group)) t = cand;
    else home_empty = true;
  }
  while (t < 0 && home_empty) {
    const int ql = (home + lane) % kNumQueues;
    int left = 0;
    if (lane < kNumQueues)
      left = atomicAdd(a.ctr + ql * kCounterStride, a.zero) < queue_units(ql, nkv, per_group);
    const unsigned long long open = __ballot(left);
    if (open == 0) break;
    q = (home + __ffsll((long long)open) - 1) % kNumQueues;
    int cand = 0;
    if (lane == 0) cand = atomicAdd(a.ctr + q * kCounterStride, 1);
    cand = __shfl(cand, 0);
    if (cand < queue_units(q, nkv, per_group)) t = cand;
  }
  t_out = t;
  q_out = q;
}

// Runs item t of queue q of the persistent schedule: maps it to its unit
// (b, hkv, hb, qb), walks the unit's key tiles and stores its rows.  All
// threads of the workgroup call it together.
// Item t of queue q of the persistent schedule -> unit (b, hkv, hb, qb).
__device__ __forceinline__ void persistent_map(const PrefillArgs& a, bool causal, int t, int q,
                                               int& b, int& hkv, int& hb, int& qb) {
  const int nkv = a.B * a.Hkv;
  const int per_group = a.HB * a.NQB;
  const int groups = queue_units(q, nkv, per_group) / per_group;
  int gi;
  if (causal) {
    const int per_qb = groups * a.HB;
    qb = a.NQB - 1 - t / per_qb;
    const int rest = t % per_qb;
    hb = rest % a.HB;
    gi = rest / a.HB;
  } else {
    gi = t / per_group;
    const int rest = t % per_group;
    hb = rest / a.NQB;
    qb = rest % a.NQB;
  }
  const int kvg = q + kNumQueues * gi;
  hkv = kvg % a.Hkv;
  b = kvg / a.Hkv;
}

template <typename T, class C, bool CAUSAL>
__device__ __forceinline__ void persistent_unit(const PrefillArgs& a, char* smem, int t, int q,
                                                int w, int j) {
  int b, hkv, hb, qb;
  persistent_map(a, CAUSAL, t, q, b, hkv, hb, qb);

  const int ntiles = unit_tiles<C, CAUSAL>(a, qb);
  const int rot = (int)((7u * (unsigned)t + 3u * (unsigned)q) % (unsigned)ntiles);
  const Column col = lane_column<C>(a, b, hkv, hb, qb, w, j);
  float mrun, lrun;
  f32x16 acc[C::DB];
  run_segment<T, C, CAUSAL>(a, smem, b, hkv, qb, 0, ntiles, rot, col, mrun, lrun, acc);
  // the ring is free (run_segment ends on a barrier); the next fetch
  // starts with a barrier before any wave writes it again
  finish_rows<T, C>(a, smem + w * stage_out_bytes<C>(), lrun, acc, b, hkv, hb, qb, w);
}

// The last workgroup to leave a persistent launch (all others have made
// their final, failing fetches) sets counters 0 .. last back to zero for
// the next launch; counter kNumQueues counts the workgroups that left.
// Wave 0 (thread 0 among its lanes) made every take and probe of its
// workgroup and used each returned value, so those atomics are complete
// before its count below is issued: no fence is needed (an agent-scope fence here writes back and invalidates the
// whole L2 at every workgroup's exit).
__device__ __forceinline__ void leave_persistent(const PrefillArgs& a, int last) {
  if (threadIdx.x == 0) {
    const int done = atomicAdd(a.ctr + kNumQueues * kCounterStride, 1);
    if (done == (int)gridDim.x - 1) {
      for (int i = 0; i <= last; ++i) atomicExch(a.ctr + i * kCounterStride, 0);
    }
  }
}

template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];
  static_assert(C::NW * stage_out_bytes<C>() <= 2 * C::STAGE_BYTES, "output staging too large");
  __shared__ int s_unit;
  __shared__ int s_queue;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;

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
    // workgroup-uniform; readfirstlane keeps what derives from them scalar
    const int t = __builtin_amdgcn_readfirstlane(s_unit);
    const int q = __builtin_amdgcn_readfirstlane(s_queue);
    if (t < 0) break;
    persistent_unit<T, C, CAUSAL>(a, smem, t, q, w, j);
  }
  leave_persistent(a, kNumQueues);
}

// Packed varlen batches (sequences of different lengths back to back in
// token-major tensors): the persistent schedule over units (sequence b,
// hkv, hb, qb) with qb below ceil(max_seqlen_q / R); a unit past its
// sequence's query rows does nothing.  Each unit runs on its own sequence:
// bases moved to the sequence's first query and key row, its own Nq and Nk,
// and, causal, its queries as its last Nq tokens (q_offset = Nk - Nq, which
// may be negative: rows that see no key come out zero).
template <typename T, class C, bool CAUSAL>
__device__ __forceinline__ void varlen_unit(const PrefillArgs& a, char* smem, int t, int q,
                                            int w, int j) {
  int b, hkv, hb, qb;
  persistent_map(a, CAUSAL, t, q, b, hkv, hb, qb);
  const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
  const int k0 = a.cu_k[b], k1 = a.cu_k[b + 1];
  const int nq = __builtin_amdgcn_readfirstlane(q1 - q0);
  const int nk = __builtin_amdgcn_readfirstlane(k1 - k0 > 0 ? k1 - k0 : 0);
  if (qb * a.R >= nq) return;  // past this sequence's queries (workgroup-uniform)
  PrefillArgs u = a;
  u.Nq = nq;
  u.Nk = nk;
  u.NQB = (nq + a.R - 1) / a.R;
  u.q_offset = CAUSAL ? nk - nq : 0;
  u.q = reinterpret_cast<const T*>(a.q) + (size_t)q0 * a.q_sn;
  u.o = reinterpret_cast<T*>(a.o) + (size_t)q0 * a.q_sn;
  const size_t kv_row = (size_t)a.kv_rowb / C::ESZ;  // elements from one key row to the next
  u.k = reinterpret_cast<const T*>(a.k) + (size_t)k0 * kv_row;
  u.v = reinterpret_cast<const T*>(a.v) + (size_t)k0 * kv_row;

  const int ntiles = nk > 0 ? unit_tiles<C, CAUSAL>(u, qb) : 0;
  const Column col = lane_column<C>(u, 0, hkv, hb, qb, w, j);
  float mrun = kNegInf, lrun = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  if (ntiles > 0) {
    const int rot = (int)((7u * (unsigned)t + 3u * (unsigned)q) % (unsigned)ntiles);
    run_segment<T, C, CAUSAL>(u, smem, 0, hkv, qb, 0, ntiles, rot, col, mrun, lrun, acc);
  }
  finish_rows<T, C>(u, smem + w * stage_out_bytes<C>(), lrun, acc, 0, hkv, hb, qb, w);
}

template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_varlen_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];
  static_assert(C::NW * stage_out_bytes<C>() <= 2 * C::STAGE_BYTES, "output staging too large");
  __shared__ int s_unit;
  __shared__ int s_queue;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;
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
    varlen_unit<T, C, CAUSAL>(a, smem, t, q, w, j);
  }
  leave_persistent(a, kNumQueues);
}

// Chunk c of slice s for workgroup g = c * nsl + s, so the workgroups of a
// slice share an XCD whenever nsl is a multiple of kNumQueues.  Segments
// that cover a whole unit store the result; a cut unit's first segment in
// the chunk goes to record slot 0 and its last to slot 1 (a segment that is
// not the chunk's first always reaches the chunk's end).  All threads of
// the workgroup call it; the LDS ring is free on return.
template <typename T, class C, bool CAUSAL>
__device__ __forceinline__ void balanced_chunk(const PrefillArgs& a, char* smem, int g) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;

  const int s = g % a.nsl;
  const int c = g / a.nsl;
  const int hb = s % a.HB;
  const int kvg = s / a.HB;
  const int hkv = kvg % a.Hkv;
  const int b = kvg / a.Hkv;

  const int x_end = chunk_bound(a, c + 1);
  int x = chunk_bound(a, c);
  int pos, pre;
  locate_tile<C, CAUSAL>(a, x, lane, pos, pre);
  for (int seg = 0; x < x_end && pos < a.NQB; ++seg) {
    const int qb = seq_qb<CAUSAL>(pos, a.NQB);
    const int n = unit_tiles<C, CAUSAL>(a, qb);
    const int t0 = x - pre;
    const int t1 = min(n, x_end - pre);
    const int ntiles = t1 - t0;
    const int rot = (int)((7u * (unsigned)g + 5u * (unsigned)seg) % (unsigned)ntiles);
    const Column col = lane_column<C>(a, b, hkv, hb, qb, w, j);
    float mrun, lrun;
    f32x16 acc[C::DB];
    run_segment<T, C, CAUSAL>(a, smem, b, hkv, qb, t0, ntiles, rot, col, mrun, lrun, acc);
    if (t0 == 0 && t1 == n) {
      finish_rows<T, C>(a, smem + w * stage_out_bytes<C>(), lrun, acc, b, hkv, hb, qb, w);
      __syncthreads();  // the staging area is ring memory again
    } else if (a.ws)  // the host provides records whenever a chunk boundary cuts a unit
      write_record<C>(part_record<C>(a, g, seg == 0 ? 0 : 1), mrun, lrun, acc, w, lane);
    x = pre + t1;
    pre += n;
    ++pos;
  }
}

// The balanced schedule: one chunk per workgroup.
template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_balanced_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];
  static_assert(C::NW * stage_out_bytes<C>() <= 2 * C::STAGE_BYTES, "output staging too large");
  balanced_chunk<T, C, CAUSAL>(a, smem, blockIdx.x);
}

// Causal launches with about one unit pair per resident workgroup: workgroup
// g of 2*NW waves runs the pair (qb = NQB-1-p, qb = p), p = g / nsl, of
// slice s = g % nsl; every pair holds about the same number of key tiles, so
// a static one-pair-per-workgroup schedule is balanced.  The units here have
// 32*NW columns (the host decomposes for that width).  The two halves of the
// workgroup (waves 0..NW-1 and NW..2NW-1) take the first and second half of
// each unit's key tiles on LDS rings of their own, for the same columns;
// the second half then hands its state (m, l, unnormalised O) to the first
// through LDS, which merges the two in a fixed order and stores the rows.
template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(2 * C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_pair_kernel(PrefillArgs a) {
  constexpr bool DK = use_direct_k<C>();
  constexpr int RING = DK ? dk_ring_bytes<C>() : 2 * C::STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * RING];
  static_assert(2 * RING >= C::NT * (C::DB * 16 + 2) * 4, "hand-over area too small");

  const int tid = threadIdx.x;
  // wave-uniform; readfirstlane keeps what derives from them scalar
  const int half = __builtin_amdgcn_readfirstlane(tid / C::NT);
  const int w = __builtin_amdgcn_readfirstlane((tid % C::NT) >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;

  const int g = blockIdx.x;
  const int s = g % a.nsl;
  const int p = g / a.nsl;
  const int hb = s % a.HB;
  const int kvg = s / a.HB;
  const int hkv = kvg % a.Hkv;
  const int b = kvg / a.Hkv;
  char* ring = smem + half * RING;
  // hand-over area: one block per wave slot w, DB*4 rows of 64 float4 (the
  // accumulator) then 64 float2 (m, l); consecutive lanes on consecutive
  // 16-byte addresses.  After the merge, wave w of the first half stages its
  // output rows in the same block.
  constexpr int HAND_BYTES = (C::DB * 16 + 2) * 64 * 4;
  static_assert(HAND_BYTES >= stage_out_bytes<C>(), "output staging exceeds the hand-over block");
  char* hand = smem + w * HAND_BYTES;
  float4* hand4 = reinterpret_cast<float4*>(hand) + lane;
  float2* hand2 = reinterpret_cast<float2*>(hand + C::DB * 4 * 64 * 16) + lane;

  // unit u of the pair (u = 1 absent for the middle unit of an odd NQB)
  const int nunits = (a.NQB - 1 - p) > p ? 2 : 1;
  auto unit_qb = [&](int u) { return u == 0 ? a.NQB - 1 - p : p; };
  auto unit_seg = [&](int u, int& n0) {
    const int n = unit_tiles<C, CAUSAL>(a, unit_qb(u));
    n0 = (n + 1) / 2;
    const int nt = half ? n - n0 : n0;
    const int rot = nt > 0 ? (int)((7u * (unsigned)g + 3u * (unsigned)u) % (unsigned)nt) : 0;
    return SegTiles{half ? min(n0, n - 1) : 0, nt, rot};
  };

  SegIn<C> in;
  int n0;
  SegTiles st = unit_seg(0, n0);
  Column col = lane_column<C>(a, b, hkv, hb, unit_qb(0), w, j);
  seg_begin<T, C, !DK>(a, in, b, hkv, st, col);
  for (int u = 0; u < nunits; ++u) {
    const int qb = unit_qb(u);
    float mrun, lrun;
    f32x16 acc[C::DB];
    if constexpr (DK)
      seg_run_direct<T, C, CAUSAL>(a, ring, in, b, hkv, qb, st, col, mrun, lrun, acc, n0);
    else
      seg_run<T, C, CAUSAL, true>(a, ring, in, b, hkv, qb, st, col, mrun, lrun, acc, n0);
    if (u + 1 < nunits) {
      // issue the next unit's Q fragment and first tiles now: their latency
      // hides behind this unit's hand-over
      st = unit_seg(u + 1, n0);
      col = lane_column<C>(a, b, hkv, hb, unit_qb(u + 1), w, j);
      seg_begin<T, C, !DK>(a, in, b, hkv, st, col);
    }
    // hand-over: the rings are free (seg_run ends on a barrier)
    if (half) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          hand4[(db * 4 + r4) * 64] = make_float4(acc[db][4 * r4], acc[db][4 * r4 + 1],
                                                  acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]);
      *hand2 = make_float2(mrun, lrun);
    }
    __syncthreads();
    if (!half) {
      const float2 ml1 = *hand2;
      const float M = fmaxf(mrun, ml1.x);
      const float w0 = mrun == kNegInf ? 0.f : fast_exp2((mrun - M) * a.c);
      const float w1 = ml1.x == kNegInf ? 0.f : fast_exp2((ml1.x - M) * a.c);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 o1 = hand4[(db * 4 + r4) * 64];
          acc[db][4 * r4] = w0 * acc[db][4 * r4] + w1 * o1.x;
          acc[db][4 * r4 + 1] = w0 * acc[db][4 * r4 + 1] + w1 * o1.y;
          acc[db][4 * r4 + 2] = w0 * acc[db][4 * r4 + 2] + w1 * o1.z;
          acc[db][4 * r4 + 3] = w0 * acc[db][4 * r4 + 3] + w1 * o1.w;
        }
      finish_rows<T, C>(a, hand, w0 * lrun + w1 * ml1.y, acc, b, hkv, hb, qb, w);
    }
    __syncthreads();  // the hand-over area is ring memory again
  }
}

// Combines the pieces of each unit cut by the balanced schedule.  Block
// (w * (Pp - 1) + c - 1) * nsl + s, of DB waves, looks at chunk boundary c of
// slice s and, if it is the first boundary inside the unit it cuts, merges
// that unit's pieces (those of chunks c - 1 .. c_hi) for the columns of
// prefill wave w; wave i of the block takes accumulator block db = i.  The
// pieces are merged in chunk order with the rescaling of the online softmax
// (piece p's state is relative to its own reference m_p; the merged
// reference is M = max_p m_p and piece p is weighted by 2^((m_p - M) c)),
// so the result does not depend on timing.  All loads of up to
// kMergeBatch pieces are issued before the first is used.
constexpr int kMergeBatch = 4;
template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(64 * C::DB) prefill_merge_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63;
  const int db = threadIdx.x >> 6;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  const int nb = a.nsl * (a.Pp - 1);
  const int w = blockIdx.x / nb;
  const int s = blockIdx.x % a.nsl;
  const int c = (blockIdx.x % nb) / a.nsl + 1;  // boundary 1 .. Pp-1
  const int X = chunk_bound(a, c);
  int pos, pre;
  locate_tile<C, CAUSAL>(a, X, lane, pos, pre);
  if (pre == X || chunk_bound(a, c - 1) > pre) return;  // no cut here, or merged elsewhere
  const int qb = seq_qb<CAUSAL>(pos, a.NQB);
  const int n = unit_tiles<C, CAUSAL>(a, qb);
  const int hb = s % a.HB;
  const int kvg = s / a.HB;
  const int hkv = kvg % a.Hkv;
  const int b = kvg / a.Hkv;
  const Column col = lane_column<C>(a, b, hkv, hb, qb, w, j);

  // pieces: chunk k = c-1 .. c_hi; chunk c-1's piece is its workgroup's
  // first segment only if the chunk starts at the unit's first tile
  int c_hi = c;
  while (c_hi + 1 < a.Pp && chunk_bound(a, c_hi + 1) < pre + n) ++c_hi;
  const int np = c_hi - c + 2;
  const int slot_first = chunk_bound(a, c - 1) < pre ? 1 : 0;
  const float* rec0 = part_record<C>(a, (c - 1) * a.nsl + s, 0) + w * wave_record_floats<C>();
  auto rec_of = [&](int p) {
    p = min(p, np - 1);  // beyond the last piece: repeat it (unused)
    return rec0 + ((size_t)p * a.nsl * 2 + (p == 0 ? slot_first : 0)) * part_floats<C>();
  };

  float2 ml[kMaxPiecesDev];
#pragma unroll
  for (int p = 0; p < kMaxPiecesDev; ++p)
    ml[p] = reinterpret_cast<const float2*>(rec_of(p) + C::DB * 16 * 64)[lane];
  float4 x[kMergeBatch][4];
#pragma unroll
  for (int p = 0; p < kMergeBatch; ++p)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      x[p][r4] = reinterpret_cast<const float4*>(rec_of(p))[(db * 4 + r4) * 64 + lane];
  float M = kNegInf;
#pragma unroll
  for (int p = 0; p < kMaxPiecesDev; ++p) M = fmaxf(M, ml[p].x);

  f32x16 acc[1] = {f32x16{}};
  float l = 0.f;
  for (int p0 = 0; p0 < np; p0 += kMergeBatch) {
    if (p0 > 0) {
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          x[p][r4] = reinterpret_cast<const float4*>(rec_of(p0 + p))[(db * 4 + r4) * 64 + lane];
    }
#pragma unroll
    for (int p = 0; p < kMergeBatch; ++p) {
      if (p0 + p < np) {
        float mp = ml[0].x, lp = ml[0].y;
#pragma unroll
        for (int i = 1; i < kMaxPiecesDev; ++i)
          if (i == p0 + p) { mp = ml[i].x; lp = ml[i].y; }
        const float wgt = mp == kNegInf ? 0.f : fast_exp2((mp - M) * a.c);
        l += wgt * lp;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          acc[0][4 * r4] += wgt * x[p][r4].x;
          acc[0][4 * r4 + 1] += wgt * x[p][r4].y;
          acc[0][4 * r4 + 2] += wgt * x[p][r4].z;
          acc[0][4 * r4 + 3] += wgt * x[p][r4].w;
        }
      }
    }
  }
  const float lsum = halves_sum(l);
  if (col.valid)
    store_out_block<T, C>(reinterpret_cast<T*>(a.o) + col.row_off, acc[0], 1.0f / lsum, db, h2);
}

// Key-split schedule for few units: one 8-wave workgroup per 64-column unit,
// as NG = 4 groups of two waves.  Group q runs the q-th quarter of the unit's
// key tiles on an LDS ring of its own; groups 1..3 then hand their states
// (m, l, unnormalised O) to group 0 through LDS, which merges the four in
// group order and stores the rows.  No partial state leaves the workgroup,
// so there is no merge pass.  Unit i / 8-th of the list runs on the XCD
// that takes block i mod 8 (when T is a multiple of 8), so the units of one
// K/V head share one L2.
template <class C>
constexpr int quad_lds_bytes() {
  return 4 * 2 * C::STAGE_BYTES;
}

// Unit t (qb = t % NQB, then head block, then K/V group) of the quad
// schedule, run by the whole 8-wave workgroup in smem (quad_lds_bytes).
// Ends with group 0 storing the rows; the caller puts a barrier between
// this and any later use of smem.
// DIRECT_OK false keeps K on the register path (the mixed launch's quad
// kernel, which was measured slower with direct K loads).
template <typename T, class C, bool CAUSAL, bool DIRECT_OK = true>
__device__ __forceinline__ void quad_unit(const PrefillArgs& a, char* smem, int t) {
  static_assert(C::NW == 2, "quad groups are two waves");
  constexpr int NG = 4;
  // hand-over block of one wave: DB*4 rows of 64 float4 (the accumulator),
  // then 64 float2 (m, l); consecutive lanes on consecutive 16-byte words
  constexpr int HAND_BYTES = (C::DB * 16 + 2) * 64 * 4;
  constexpr int STAGE_OFF = (NG - 1) * C::NW * HAND_BYTES;
  static_assert(STAGE_OFF + C::NW * stage_out_bytes<C>() <= NG * 2 * C::STAGE_BYTES,
                "hand-over and output staging exceed the rings");

  const int tid = threadIdx.x;
  // wave-uniform; readfirstlane keeps what derives from them scalar
  const int grp = __builtin_amdgcn_readfirstlane(tid / C::NT);
  const int w = __builtin_amdgcn_readfirstlane((tid % C::NT) >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;

  const int qb = t % a.NQB;
  const int rest = t / a.NQB;
  const int hb = rest % a.HB;
  const int kvg = rest / a.HB;
  const int hkv = kvg % a.Hkv;
  const int b = kvg / a.Hkv;

  const int n = unit_tiles<C, CAUSAL>(a, qb);  // >= 1
  const int q0 = n * grp / NG;
  const int nt = n * (grp + 1) / NG - q0;
  const int steps = (n + NG - 1) / NG;  // the longest group range
  const int rot = nt > 0 ? (int)((7u * (unsigned)t + 3u * (unsigned)grp) % (unsigned)nt) : 0;
  const SegTiles st{min(q0, n - 1), nt, rot};
  const Column col = lane_column<C>(a, b, hkv, hb, qb, w, j);

  SegIn<C> in;
  constexpr bool DK = DIRECT_OK && use_direct_k<C>();
  static_assert(!DK || dk_ring_bytes<C>() <= 2 * C::STAGE_BYTES, "direct-K ring exceeds a group's");
  seg_begin<T, C, !DK>(a, in, b, hkv, st, col);
  float mrun, lrun;
  f32x16 acc[C::DB];
  if constexpr (DK)
    seg_run_direct<T, C, CAUSAL>(a, smem + grp * 2 * C::STAGE_BYTES, in, b, hkv, qb, st, col,
                                 mrun, lrun, acc, steps);
  else
    seg_run<T, C, CAUSAL, true>(a, smem + grp * 2 * C::STAGE_BYTES, in, b, hkv, qb, st, col,
                                mrun, lrun, acc, steps);
  // seg_run ends on a barrier: every ring is free
  if (grp > 0) {
    char* hand = smem + ((grp - 1) * C::NW + w) * HAND_BYTES;
    float4* hand4 = reinterpret_cast<float4*>(hand) + lane;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        hand4[(db * 4 + r4) * 64] = make_float4(acc[db][4 * r4], acc[db][4 * r4 + 1],
                                                acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]);
    reinterpret_cast<float2*>(hand + C::DB * 4 * 64 * 16)[lane] = make_float2(mrun, lrun);
  }
  __syncthreads();
  if (grp == 0) {
    float2 ml[NG - 1];
#pragma unroll
    for (int q = 1; q < NG; ++q)
      ml[q - 1] = reinterpret_cast<const float2*>(smem + ((q - 1) * C::NW + w) * HAND_BYTES +
                                                  C::DB * 4 * 64 * 16)[lane];
    float M = mrun;
#pragma unroll
    for (int q = 1; q < NG; ++q) M = fmaxf(M, ml[q - 1].x);
    // a state whose keys were all masked (m = -inf) has nothing to add
    const float w0 = mrun == kNegInf ? 0.f : fast_exp2((mrun - M) * a.c);
    float l = w0 * lrun;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= w0;
#pragma unroll
    for (int q = 1; q < NG; ++q) {
      const float wq = ml[q - 1].x == kNegInf ? 0.f : fast_exp2((ml[q - 1].x - M) * a.c);
      l += wq * ml[q - 1].y;
      const float4* h4 =
          reinterpret_cast<const float4*>(smem + ((q - 1) * C::NW + w) * HAND_BYTES) + lane;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 o = h4[(db * 4 + r4) * 64];
          acc[db][4 * r4] += wq * o.x;
          acc[db][4 * r4 + 1] += wq * o.y;
          acc[db][4 * r4 + 2] += wq * o.z;
          acc[db][4 * r4 + 3] += wq * o.w;
        }
    }
    finish_rows<T, C>(a, smem + STAGE_OFF + w * stage_out_bytes<C>(), l, acc, b, hkv, hb, qb,
                      w);
  }
}

template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(4 * C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_quad_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[quad_lds_bytes<C>()];
  const int i = blockIdx.x;
  const int t = (a.T % 8 == 0) ? (i % 8) * (a.T / 8) + i / 8 : i;
  quad_unit<T, C, CAUSAL>(a, smem, t);
}

}  // namespace gqa
