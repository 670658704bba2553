// prefill_kernel.hpp -- persistent GQA forward (prefill and chunked prefill).
//
// Work unit = (batch b, K/V head hkv, head block hb, position block qb): the
// Gu query heads hb*Gu .. hb*Gu+Gu-1 of the group that shares K/V head hkv
// (head mapping hkv = h / g, BootstrapAI evolution log, "Kernel 9 -- GQA"),
// stacked over R consecutive query positions, Gu*R <= 32*NW columns.  Column
// m of the unit is head r = m / R at position p = m % R, so every K/V tile a
// workgroup stages in LDS is read from HBM once and serves all Gu heads: the
// "one K/V tile shared by many query rows" idea of the same log's
// cooperative-loading kernel ("Kernel 3"), widened from query rows to the
// whole head group.
//
// Scheduling is persistent ("Kernel 8 -- persistent kernel" of the same
// log): the grid holds as many workgroups as fit on the device at once and
// each repeatedly takes the next unit from a device counter with one atomic
// add, exiting once every unit is taken.  The units are split into
// kNumQueues queues by K/V group (b*Hkv + hkv) modulo kNumQueues, one per
// XCD: workgroups are dispatched to the XCDs round-robin by block index, so
// a workgroup first drains the queue of its own XCD and the K/V tiles of a
// group stay in that XCD's L2; a workgroup whose queue is empty steals from
// the next ones.  Within a queue units are numbered heaviest first for
// causal attention (the last position blocks see the most keys), which
// makes the first-come order a longest-job-first schedule; for non-causal
// attention the units of one K/V group are numbered consecutively.  The
// last workgroup to leave resets the counters for the next launch.
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
  int g;    // Hq / Hkv
  int Gu;   // query heads per unit
  int R;    // query positions per unit
  int HB;   // head blocks per K/V head, ceil(g / Gu)
  int NQB;  // position blocks, ceil(Nq / R)
  int T;    // units, B * Hkv * HB * NQB
  int q_offset;
  float c;  // |scale| * log2(e)
  int negate_q;
  int* ctr;  // [0, kNumQueues): next unit of each queue; [kNumQueues]: workgroups finished
};

constexpr int kNumQueues = 8;  // XCDs of an MI355X

// Units in queue q: the K/V groups q, q + kNumQueues, ... below nkv.
__device__ __forceinline__ int queue_units(int q, int nkv, int per_group) {
  return nkv > q ? ((nkv - q + kNumQueues - 1) / kNumQueues) * per_group : 0;
}

template <typename T, class C, bool CAUSAL>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2)))
prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];
  __shared__ int s_unit;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // stage st: K at smem + st*STAGE_BYTES, V right after it
  auto stK = [&](int st) { return reinterpret_cast<T*>(smem + st * C::STAGE_BYTES); };
  auto stV = [&](int st) { return stK(st) + C::K_ELEMS; };

  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ K = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ V = reinterpret_cast<const T*>(a.v);
  T* __restrict__ O = reinterpret_cast<T*>(a.o);

  __shared__ int s_queue;
  const int home = blockIdx.x % kNumQueues;
  const int nkv = a.B * a.Hkv;
  const int per_group = a.HB * a.NQB;
  int tried = 0;  // queues found empty so far (thread 0 only)

  for (;;) {
    if (tid == 0) {
      int t = -1, q = 0;
      while (tried < kNumQueues) {
        q = (home + tried) % kNumQueues;
        const int cand = atomicAdd(a.ctr + q, 1);
        if (cand < queue_units(q, nkv, per_group)) {
          t = cand;
          break;
        }
        ++tried;
      }
      s_unit = t;
      s_queue = q;
    }
    __syncthreads();
    const int t = s_unit;
    const int q = s_queue;
    if (t < 0) break;

    // ---- (queue, index) -> (b, hkv, hb, qb)
    const int groups = queue_units(q, nkv, per_group) / per_group;
    int qb, gi, hb;
    if (CAUSAL) {
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
    const int hkv = kvg % a.Hkv;
    const int b = kvg / a.Hkv;

    // ---- this lane's query column
    const int m = 32 * w + j;
    const int r = m / a.R;
    const int p = m - r * a.R;
    const int hig = hb * a.Gu + r;  // head within the group
    const int i = qb * a.R + p;     // query row
    const bool valid = (r < a.Gu) && (hig < a.g) && (i < a.Nq);
    const int h = hkv * a.g + hig;
    const size_t qrow_off = valid ? (((size_t)b * a.Hq + h) * a.Nq + i) * C::D : 0;

    typename C::Frag qf[C::QF];
    load_q_frag<T, C>(qf, Q + qrow_off, valid, a.negate_q != 0, h2);

    const size_t kv_off = ((size_t)b * a.Hkv + hkv) * a.Nk * C::D;
    const T* kbase = K + kv_off;
    const T* vbase = V + kv_off;

    // ---- key range of the unit
    const int i_lo = qb * a.R;
    const int i_hi = min(a.Nq, i_lo + a.R) - 1;
    const int kend = CAUSAL ? min(a.Nk, a.q_offset + i_hi + 1) : a.Nk;
    const int ntiles = (kend + C::BC - 1) / C::BC;
    // keys below full_lim are visible to every column of the unit
    const int full_lim = CAUSAL ? min(a.Nk, a.q_offset + i_lo + 1) : a.Nk;
    // last key this lane's query may see
    const int lim = (CAUSAL && valid) ? min(a.q_offset + i, a.Nk - 1) : a.Nk - 1;

    float mrun = kNegInf, lrun = 0.f;
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    // Two LDS stages and two register staging sets: the global loads of tile
    // t+2 are issued at the start of tile t and written to LDS at the end of
    // tile t+1, so two tiles of compute cover their latency.  The loop is
    // unrolled by two so each staging set is a named register set, and the
    // loads and stores are unconditional (indices clamped to the last tile)
    // so the compiler's wait before each LDS store counts exactly the newer
    // loads still in flight.
    //
    // Each unit walks its tiles starting at a unit-dependent rotation, so the
    // many workgroups that share a K/V head do not all request the same
    // tile at the same moment.  The order of tiles does not change the
    // result in exact arithmetic (masking is per key, and a lane whose first
    // tiles are all masked keeps an empty state until a visible key comes).
    const int rot = (int)((7u * (unsigned)t + 3u * (unsigned)q) % (unsigned)ntiles);
    auto tile_at = [&](int pos) {
      const int x = (pos < ntiles ? pos : ntiles - 1) + rot;
      return x >= ntiles ? x - ntiles : x;
    };
    TileRegs<C> ra, rb;
    load_tile<T, C>(ra, kbase, vbase, tile_at(0) * C::BC, a.Nk, tid);
    load_tile<T, C>(rb, kbase, vbase, tile_at(1) * C::BC, a.Nk, tid);
    store_tile<T, C>(ra, stK(0), stV(0), tid);
    __syncthreads();

    auto step = [&](TileRegs<C>& mine, TileRegs<C>& next, int kt) {
      const int cur = kt & 1;
      load_tile<T, C>(mine, kbase, vbase, tile_at(kt + 2) * C::BC, a.Nk, tid);
      f32x16 s[C::KB];
      qk_tile<T, C>(s, qf, stK(cur), j, h2);
      const int key0 = tile_at(kt) * C::BC;
      if (key0 + C::BC > full_lim) mask_tile<C>(s, key0, lim, h2);
      softmax_pv_step<T, C>(s, mrun, lrun, acc, stV(cur), j, h2, a.c);
      store_tile<T, C>(next, stK(cur ^ 1), stV(cur ^ 1), tid);
      __syncthreads();
    };
    for (int kt = 0; kt < ntiles; kt += 2) {
      step(ra, rb, kt);
      if (kt + 1 < ntiles) step(rb, ra, kt + 1);
    }

    const float lsum = lrun + __shfl_xor(lrun, 32);
    if (valid) store_out_row<T, C>(O + qrow_off, acc, 1.0f / lsum, h2);
  }

  // Leave the counters at zero for the next launch: the last workgroup out
  // (all others have made their final, failing fetches) resets every word.
  if (tid == 0) {
    __threadfence();
    const int done = atomicAdd(a.ctr + kNumQueues, 1);
    if (done == (int)gridDim.x - 1) {
      for (int i = 0; i <= kNumQueues; ++i) atomicExch(a.ctr + i, 0);
    }
  }
}

}  // namespace gqa
