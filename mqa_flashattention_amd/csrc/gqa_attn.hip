// gqa_attn.hip -- the C ABI of libgqa_attn.so (declared in include/gqa_attn.h).
//
// Host side only: argument validation (pure CPU, before any HIP call), the
// gfx950 device check, the per-(device, stream) scheduler counters, choice
// of the unit decomposition and split size, and the kernel launches.  All
// arithmetic runs in the kernels of prefill_kernel.hpp / decode_kernel.hpp /
// mixed_kernel.hpp / backward_kernel.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "backward_kernel.hpp"
#include "decode_kernel.hpp"
#include "decode_part.hpp"
#include "gqa_attn.h"
#include "mixed_kernel.hpp"
#include "prefill_kernel.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

// |scale| * log2(e), floored at 1e-30: the kernels need a positive factor
// (masked scores are -inf and must give weight exp2(-inf) = 0).  For a zero
// scale every |score - max| * 1e-30 is below 2^-24, so each weight is exactly
// 1 and the result is the plain mean, as the definition says.
float softmax_coef(float scale) {
  const float c = std::fabs(scale) * gqa::kLog2e;
  return c > 1e-30f ? c : 1e-30f;
}

constexpr long long kIntMax = 2147483647LL;

struct DeviceInfo {
  bool gfx950 = false;
  int cus = 0;
  std::string arch;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_devices;
std::map<const void*, int> g_occupancy;

// The current device, checked to be a gfx950.
int current_device(int* dev_out, DeviceInfo* info_out) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(GQA_ERR_NO_DEVICE, "no HIP device available (%s)",
                e == hipSuccess ? "device count is 0" : hipGetErrorString(e));
  }
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_devices.find(dev);
  if (it == g_devices.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    DeviceInfo info;
    info.arch = prop.gcnArchName;
    info.gfx950 = info.arch.compare(0, 6, "gfx950") == 0;
    info.cus = prop.multiProcessorCount;
    it = g_devices.emplace(dev, info).first;
  }
  if (!it->second.gfx950)
    return fail(GQA_ERR_NO_DEVICE, "device %d is %s, this library runs on gfx950 only", dev,
                it->second.arch.c_str());
  *dev_out = dev;
  *info_out = it->second;
  return GQA_OK;
}

__global__ void zero_ints_kernel(int* p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t zero_ints(int* p, long long n, hipStream_t stream) {
  long long blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// Device memory the library keeps per (device, stream):
//  * ctr: one counter per work queue, a finished-workgroup count and the
//    mixed launch's decode-split counter, zeroed in stream order when
//    allocated; each persistent launch leaves them at zero when it ends;
//  * ws: partial records of the prefill units that the balanced schedule
//    cuts, grown on demand to at least twice its size.  A replaced buffer is
//    kept, not freed, until the process ends: launches still queued, and
//    HIP graphs captured earlier, keep using it.
// Neither may be set up while the stream is being captured into a HIP graph
// (an allocation is not graph work): such a call fails, and one eager call
// with the same sizes on the stream beforehand makes the captured one
// allocation-free.
constexpr int kCounterInts = (gqa::kMixedDecodeCounter + 1) * gqa::kCounterStride;
struct StreamState {
  int* ctr = nullptr;
  float* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<void*> retired;  // replaced record buffers (see above)
};
std::map<std::pair<int, void*>, StreamState> g_streams;

int stream_state(int dev, hipStream_t stream, size_t ws_bytes, StreamState* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  StreamState& s = g_streams[std::make_pair(dev, reinterpret_cast<void*>(stream))];
  hipError_t e;
  if (!s.ctr || ws_bytes > s.ws_bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(GQA_ERR_UNSUPPORTED,
                  "this call would set up the stream's scheduler state (%s) while the stream "
                  "is captured; make one call with the same sizes on this stream before capture",
                  !s.ctr ? "first call on the stream" : "larger split workspace");
  }
  if (!s.ctr) {
    e = hipMalloc(&s.ctr, kCounterInts * sizeof(int));
    if (e != hipSuccess) {
      s.ctr = nullptr;
      return hip_fail(e, "hipMalloc(scheduler counters)");
    }
    e = zero_ints(s.ctr, kCounterInts, stream);
    if (e != hipSuccess) {
      (void)hipFree(s.ctr);
      s.ctr = nullptr;
      return hip_fail(e, "counter initialisation launch");
    }
  }
  if (ws_bytes > s.ws_bytes) {
    const size_t grow = std::max(ws_bytes, 2 * s.ws_bytes);
    float* fresh = nullptr;
    e = hipMalloc(&fresh, grow);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(split workspace)");
    if (s.ws) s.retired.push_back(s.ws);
    s.ws = fresh;
    s.ws_bytes = grow;
  }
  out->ctr = s.ctr;
  out->ws = s.ws;
  out->ws_bytes = s.ws_bytes;
  return GQA_OK;
}

// Resident workgroups per CU of a kernel (cached).
int occupancy(const void* kernel, int threads) {
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_occupancy.find(kernel);
    if (it != g_occupancy.end()) return it->second;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess ||
      nb < 1) {
    (void)hipGetLastError();
    nb = 1;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  g_occupancy[kernel] = nb;
  return nb;
}

// ------------------------------------------------------------------ prefill

// bf16: 32-key tiles at d=128 (two register staging sets fit the budget of
// two waves per SIMD), 64-key tiles below; fp32: 32-key tiles.  Four waves
// per workgroup, 128 query columns per unit.
constexpr int kPrefillWaves = 4;
constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU
template <int D>
using CfgBf16 = gqa::TileCfg<uint16_t, D, (D == 128 ? 32 : 64), kPrefillWaves>;
template <int D>
using CfgF32 = gqa::TileCfg<float, D, 32, kPrefillWaves>;
// the same with a run-time K/V key-row stride (token-major or padded K/V)
template <int D>
using CfgBf16S = gqa::TileCfg<uint16_t, D, (D == 128 ? 32 : 64), kPrefillWaves, true>;
template <int D>
using CfgF32S = gqa::TileCfg<float, D, 32, kPrefillWaves, true>;

// Unit decomposition for units of M columns: Gu = min(g, M) heads of a
// group stacked over R = M / Gu positions, HB head blocks per group, NQB
// position blocks, T units.
void decompose(gqa::PrefillArgs& a, int M) {
  a.Gu = a.g < M ? a.g : M;
  a.R = M / a.Gu;
  a.HB = (a.g + a.Gu - 1) / a.Gu;
  a.NQB = a.Nq > 0 ? (a.Nq - 1) / a.R + 1 : 0;
  // callers reject sizes past INT_MAX units; the clamp only keeps this
  // product defined before they look
  const long long T = (long long)a.B * a.Hkv * a.HB * a.NQB;
  a.T = (int)std::min<long long>(T, kIntMax);
}

// Key tiles of the units of position block qb (host copy of the kernels'
// unit_tiles).
template <class C>
long long unit_tiles(const gqa::PrefillArgs& a, bool causal, long long qb) {
  long long kend = a.Nk;
  if (causal) {
    const long long i_hi = std::min<long long>(a.Nq, (qb + 1) * a.R) - 1;
    kend = std::min<long long>(a.Nk, a.q_offset + i_hi + 1);
  }
  return (kend + C::BC - 1) / C::BC;
}

long long seq_qb(long long pos, long long nqb, bool causal) {
  if (!causal) return pos;
  return (pos & 1) ? (pos >> 1) : nqb - 1 - (pos >> 1);
}

// The balanced schedule (a static partition of each slice's key tiles into
// Pp equal chunks, one workgroup each, plus a merge of the units the chunk
// boundaries cut) replaces the persistent one when there are too few units
// to balance whole units: at most kBalancedUnitsPerSlot per resident
// workgroup.  Pp is as large as the resident workgroups allow, but no chunk
// is shorter than kMinChunkTiles and no unit is cut into more than
// kMaxPieces pieces.  Returns false (persistent schedule) otherwise;
// *cuts is the number of units that need merging.  Each piece of a cut unit
// costs a prologue, a partial record written and read back, and a place in
// the merge; chunks of at least 8 tiles were measured faster than 4-tile
// ones (non-causal 1024 x 1024 with 64 units: 26.6 against 33.7 us) and no
// slower elsewhere by more than 3 %.
constexpr int kBalancedUnitsPerSlot = 2;
constexpr int kMinChunkTiles = 8;
constexpr int kMaxPieces = gqa::kMaxPiecesDev;
template <class C>
bool plan_balanced(gqa::PrefillArgs& a, bool causal, long long slots, long long* cuts) {
  a.nsl = a.B * a.Hkv * a.HB;
  a.Pp = 1;
  a.Ws = 0;
  *cuts = 0;
  if ((long long)a.T > kBalancedUnitsPerSlot * slots || a.nsl > slots) return false;
  long long ws = 0, longest = 0;
  for (long long qb = 0; qb < a.NQB; ++qb) {
    const long long n = unit_tiles<C>(a, causal, qb);
    ws += n;
    longest = std::max(longest, n);
  }
  if (ws > kIntMax / 2) return false;
  long long pp = slots / a.nsl;
  pp = std::min(pp, std::max<long long>(1, ws / kMinChunkTiles));
  pp = std::min(pp, std::max<long long>(1, (kMaxPieces - 1) * ws / longest));
  if (pp < 1) pp = 1;
  a.Pp = (int)pp;
  a.Ws = (int)ws;
  // count the units cut by a chunk boundary (each counted once)
  long long pre = 0, c = 1;
  for (long long pos = 0; pos < a.NQB && c < pp; ++pos) {
    const long long n = unit_tiles<C>(a, causal, seq_qb(pos, a.NQB, causal));
    bool cut = false;
    for (; c < pp; ++c) {
      const long long x = c * ws / pp;
      if (x >= pre + n) break;
      if (x > pre) cut = true;
    }
    if (cut) ++*cuts;
    pre += n;
  }
  *cuts *= a.nsl;
  return true;
}

template <typename T, class C, bool CAUSAL>
int launch_prefill(gqa::PrefillArgs& a, int dev_id, const DeviceInfo& dev, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(&gqa::prefill_kernel<T, C, CAUSAL>);
  const int per_cu = occupancy(kern, C::NT);
  const long long slots = (long long)dev.cus * per_cu;
  // Fewer 128-column units than CUs, but 3/4 to 1 of them per CU as
  // 64-column units with >= 8 key tiles each: one 8-wave workgroup per
  // 64-column unit whose four 2-wave groups split the unit's keys and merge
  // in LDS -- no partial records, no merge pass.  (Needs eight 2-wave ring
  // stages in LDS.)
  using CQ = gqa::TileCfg<T, C::D, C::BC, 2, C::KVS>;
  if constexpr (8 * CQ::STAGE_BYTES <= kLdsBytes) {
    gqa::PrefillArgs q = a;
    decompose(q, 64);
    const long long t64 = q.T;
    const long long min_tiles = unit_tiles<CQ>(q, CAUSAL, 0);  // the lightest unit
    if (a.T < dev.cus && 4 * t64 >= 3LL * dev.cus && t64 <= dev.cus && min_tiles >= 8) {
      (void)hipGetLastError();  // a stale error belongs to an earlier call
      hipLaunchKernelGGL((gqa::prefill_quad_kernel<T, CQ, CAUSAL>), dim3((unsigned)t64),
                         dim3(4 * CQ::NT), 0, stream, q);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "prefill quad kernel launch");
      return GQA_OK;
    }
  }
  long long cuts = 0;
  const bool balanced = plan_balanced<C>(a, CAUSAL, slots, &cuts);
  // causal, with at least one heavy/light unit pair per CU: one pair per
  // workgroup of two 4-wave halves that split each unit's keys.  (Halves
  // of 2 waves on 64-column units, two workgroups per CU, were measured
  // slower: each staged tile then serves half as many columns.)
  if constexpr (CAUSAL) {
    using CP = C;
    gqa::PrefillArgs p = a;
    long long pairs = 0;
    if (balanced) {
      decompose(p, 32 * CP::NW);
      p.nsl = p.B * p.Hkv * p.HB;
      pairs = (long long)p.nsl * ((p.NQB + 1) / 2);
    }
    if (balanced && pairs >= dev.cus) {  // (no counters, no workspace)
      (void)hipGetLastError();  // a stale error belongs to an earlier call
      hipLaunchKernelGGL((gqa::prefill_pair_kernel<T, CP, CAUSAL>), dim3((unsigned)pairs),
                         dim3(2 * CP::NT), 0, stream, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "prefill pair kernel launch");
      return GQA_OK;
    }
  }
  const long long grid = balanced ? (long long)a.nsl * a.Pp : std::min<long long>(a.T, slots);
  const size_t ws_bytes = cuts > 0 ? (size_t)grid * 2 * gqa::part_floats<C>() * sizeof(float) : 0;
  StreamState ss;
  int st = stream_state(dev_id, stream, ws_bytes, &ss);
  if (st != GQA_OK) return st;
  a.ctr = ss.ctr;
  a.zero = 0;
  a.ws = cuts > 0 ? ss.ws : nullptr;
  (void)hipGetLastError();  // a stale error belongs to an earlier call
  if (!balanced) {
    hipLaunchKernelGGL((gqa::prefill_kernel<T, C, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return GQA_OK;
  }
  hipLaunchKernelGGL((gqa::prefill_balanced_kernel<T, C, CAUSAL>), dim3((unsigned)grid),
                     dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
  if (cuts > 0) {
    hipLaunchKernelGGL((gqa::prefill_merge_kernel<T, C, CAUSAL>),
                       dim3((unsigned)(a.nsl * (a.Pp - 1) * C::NW)), dim3(64 * C::DB), 0, stream,
                       a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "prefill merge kernel launch");
  }
  return GQA_OK;
}

template <typename T, int D, template <int> class Cfg>
int dispatch_prefill_d(gqa::PrefillArgs& a, int causal, int dev_id, const DeviceInfo& dev,
                       hipStream_t s) {
  return causal ? launch_prefill<T, Cfg<D>, true>(a, dev_id, dev, s)
                : launch_prefill<T, Cfg<D>, false>(a, dev_id, dev, s);
}

template <typename T, template <int> class Cfg>
int dispatch_prefill(gqa::PrefillArgs& a, int d, int causal, int dev_id,
                     const DeviceInfo& dev, hipStream_t s) {
  switch (d) {
    case 32: return dispatch_prefill_d<T, 32, Cfg>(a, causal, dev_id, dev, s);
    case 64: return dispatch_prefill_d<T, 64, Cfg>(a, causal, dev_id, dev, s);
    default: return dispatch_prefill_d<T, 128, Cfg>(a, causal, dev_id, dev, s);
  }
}

// ------------------------------------------------------------------ static scratch

// Scratch of gqa_attn_decode_noalloc, for callers that cannot allocate: the
// split records of one decode call, in a file-scope device array.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: host code
// uses only the address hipGetSymbolAddress returns for the current device
// (kept per device by scratch_address), never the array's name.
constexpr size_t kNoAllocScratchBytes = GQA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::map<int, void*> g_scratch;  // device -> address of its copy of `scratch`

// The address of `scratch` on device dev, which must be the current device.
int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "hipGetSymbolAddress(static decode scratch)");
    }
    it = g_scratch.emplace(dev, p).first;
  }
  *out = it->second;
  return GQA_OK;
}

// ------------------------------------------------------------------ packed varlen

// The persistent schedule over (sequence, K/V head, head block, position
// block < ceil(max_seqlen_q / R)) units; units past a sequence's query rows
// return at once.
template <typename T, class C, bool CAUSAL>
int launch_varlen(gqa::PrefillArgs& a, int dev_id, const DeviceInfo& dev, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(&gqa::prefill_varlen_kernel<T, C, CAUSAL>);
  const long long slots = (long long)dev.cus * occupancy(kern, C::NT);
  const long long grid = std::min<long long>(a.T, slots);
  StreamState ss;
  int st = stream_state(dev_id, stream, 0, &ss);
  if (st != GQA_OK) return st;
  a.ctr = ss.ctr;
  a.zero = 0;
  a.ws = nullptr;
  (void)hipGetLastError();  // a stale error belongs to an earlier call
  hipLaunchKernelGGL((gqa::prefill_varlen_kernel<T, C, CAUSAL>), dim3((unsigned)grid),
                     dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill varlen kernel launch");
  return GQA_OK;
}

template <typename T, template <int> class Cfg>
int dispatch_varlen(gqa::PrefillArgs& a, int d, int causal, int dev_id, const DeviceInfo& dev,
                    hipStream_t s) {
  switch (d) {
    case 32:
      return causal ? launch_varlen<T, Cfg<32>, true>(a, dev_id, dev, s)
                    : launch_varlen<T, Cfg<32>, false>(a, dev_id, dev, s);
    case 64:
      return causal ? launch_varlen<T, Cfg<64>, true>(a, dev_id, dev, s)
                    : launch_varlen<T, Cfg<64>, false>(a, dev_id, dev, s);
    default:
      return causal ? launch_varlen<T, Cfg<128>, true>(a, dev_id, dev, s)
                    : launch_varlen<T, Cfg<128>, false>(a, dev_id, dev, s);
  }
}

int varlen_entry(const void* q, const void* k, const void* v, void* o, const int32_t* cu_q,
                 const int32_t* cu_k, int nseq, int max_seqlen_q, int Hq, int Hkv, int d,
                 int causal, float scale, int dtype, void* stream) {
  // ---- validation: host only, before any HIP call
  if (!q || !k || !v || !o || !cu_q || !cu_k)
    return fail(GQA_ERR_NULL_POINTER, "q, k, v, o, cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (nseq < 1 || max_seqlen_q < 1 || Hq < 1 || Hkv < 1 || d < 1)
    return fail(GQA_ERR_BAD_SHAPE,
                "sizes must be >= 1 (nseq=%d max_seqlen_q=%d Hq=%d Hkv=%d d=%d)", nseq,
                max_seqlen_q, Hq, Hkv, d);
  if (max_seqlen_q > (1 << 30))
    return fail(GQA_ERR_BAD_SHAPE, "max_seqlen_q=%d above 2^30", max_seqlen_q);
  if (Hq % Hkv != 0)
    return fail(GQA_ERR_HEAD_GROUPING, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (!std::isfinite(scale)) return fail(GQA_ERR_UNSUPPORTED, "scale must be finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(GQA_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u))
    return fail(GQA_ERR_UNSUPPORTED, "offset arrays must be 4-byte aligned");
  const int esz = dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if ((long long)Hkv * d * esz * 64 > kIntMax)
    return fail(GQA_ERR_BAD_SHAPE, "too many K/V heads for 32-bit tile offsets");
  gqa::PrefillArgs a = gqa::PrefillArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.B = nseq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = max_seqlen_q;
  a.Nk = 0;  // per sequence, on the device
  // token-major [token, head, d]: the batch index of a unit is its sequence,
  // whose rows the kernel reaches through the offset arrays
  a.q_sb = 0;
  a.q_sh = d;
  a.q_sn = (long long)Hq * d;
  a.kv_sb = 0;
  a.kv_sh = d;
  a.kv_rowb = Hkv * d * esz;
  a.g = Hq / Hkv;
  decompose(a, 32 * kPrefillWaves);
  const long long T = (long long)nseq * Hkv * a.HB * (((long long)max_seqlen_q + a.R - 1) / a.R);
  if (T > kIntMax) return fail(GQA_ERR_BAD_SHAPE, "too many work units (%lld)", T);
  a.q_offset = 0;
  a.c = softmax_coef(scale);
  a.thr = gqa::kRescaleSlack / a.c;
  a.negate_q = scale < 0.f ? 1 : 0;
  a.cu_q = cu_q;
  a.cu_k = cu_k;

  int dev = 0;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != GQA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (dtype == GQA_DTYPE_BF16) return dispatch_varlen<uint16_t, CfgBf16S>(a, d, causal, dev, info, hs);
  return dispatch_varlen<float, CfgF32S>(a, d, causal, dev, info, hs);
}

// ------------------------------------------------------------------ decode

constexpr int kMinSplit = 32;

template <int D>
using DecCfgBf16 = gqa::TileCfg<uint16_t, D, 32, 1>;
template <int D>
using DecCfgF32 = gqa::TileCfg<float, D, 32, 1>;

// Tokens per split: enough splits to put one wave on every SIMD (four per
// CU) when every row is full, in whole 32-token tiles.  The split kernel's
// registers allow one resident wave per SIMD; more, shorter splits only run
// in a second round (measured slower from batch 32 up, as were two waves
// per CU).  The mixed launch, whose decode waves hold one register stage,
// sizes its splits for eight waves per CU (waves_per_cu = 8) when its
// prefill units fill the device.
int decode_split_tokens(int B, int Hkv, int ncb, int smax, int cus, int waves_per_cu = 4) {
  const long long tiles_per_row = (smax + 31) / 32;
  const long long heads = (long long)B * Hkv * ncb;
  const long long target = (long long)waves_per_cu * cus;
  long long tiles_per_split = (heads * tiles_per_row + target - 1) / target;
  if (tiles_per_split < 1) tiles_per_split = 1;
  if (tiles_per_split > tiles_per_row) tiles_per_split = tiles_per_row;
  return (int)(tiles_per_split * 32);
}

template <typename T, class C, bool APPEND>
int launch_decode(gqa::DecodeArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.NS, (unsigned)(a.Hkv * a.NCB), (unsigned)a.B);
  hipLaunchKernelGGL((gqa::decode_split_kernel<T, C, APPEND>), grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode split kernel launch");
  hipLaunchKernelGGL((gqa::decode_combine_kernel<T, C::D, APPEND>),
                     dim3((unsigned)a.Hq, (unsigned)a.B), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode combine kernel launch");
  return GQA_OK;
}

template <typename T, template <int> class Cfg, bool APPEND>
int dispatch_decode(gqa::DecodeArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 32: return launch_decode<T, Cfg<32>, APPEND>(a, s);
    case 64: return launch_decode<T, Cfg<64>, APPEND>(a, s);
    default: return launch_decode<T, Cfg<128>, APPEND>(a, s);
  }
}

// bf16 decode (decode_part.hpp): one workgroup of W waves per (part, K/V
// head, column group, row), its waves on interleaved 32-token tiles of the
// part, merged through LDS into one record per query head; the merge kernel
// then combines a row's records.  Waves hold 16 query columns per block:
// one block for groups of up to 16 heads, two above (in ceil(g / (16 NCB))
// column groups).  The part length aims for about kPartWavesPerCu waves per
// CU when every row is full -- several rounds of workgroups, which the
// dispatcher balances over rows of different lengths -- and at most
// kPartMaxParts parts per row.
#ifndef GQA_PART_W
#define GQA_PART_W 4
#endif
#ifndef GQA_PART_WAVES_PER_CU
#define GQA_PART_WAVES_PER_CU 8
#endif
constexpr int kPartMaxParts = 64;     // records per row the merge kernel reads at once
constexpr int kPartWavesPerCu = GQA_PART_WAVES_PER_CU;

template <int D, int NCB>
using PartCfgOf = gqa::PartCfg<D, NCB, NCB == 1 ? GQA_PART_W : (GQA_PART_W > 1 ? GQA_PART_W / 2 : 1)>;

// Column groups and part length of a bf16 decode (sets a.NCB, a.S_TOK, a.NS).
template <class P>
void part_plan(gqa::DecodeArgs& a, int cus) {
  const long long ncg = (a.g + P::COLS - 1) / P::COLS;
  const long long tiles_row = (a.Smax + 31) / 32;
  const long long tiles = (long long)a.B * a.Hkv * ncg * tiles_row;
  const long long target = (long long)kPartWavesPerCu * cus;
  long long tw = (tiles + target - 1) / target;
  const long long tw_min = (tiles_row + (long long)kPartMaxParts * P::W - 1) /
                           ((long long)kPartMaxParts * P::W);
  tw = std::max(std::max(tw, tw_min), 1LL);
  a.NCB = (int)ncg;
  a.S_TOK = (int)std::min<long long>(tw * P::W * 32, kIntMax);
  a.NS = (int)((a.Smax + (long long)a.S_TOK - 1) / a.S_TOK);
}

template <int D, int NCB, bool APPEND>
int launch_decode_part(gqa::DecodeArgs& a, int cus, hipStream_t stream) {
  using P = PartCfgOf<D, NCB>;
  part_plan<P>(a, cus);
  dim3 grid((unsigned)a.NS, (unsigned)(a.Hkv * a.NCB), (unsigned)a.B);
  hipLaunchKernelGGL((gqa::decode_part_kernel<P, APPEND>), grid, dim3(P::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode part kernel launch");
  hipLaunchKernelGGL((gqa::decode_merge_kernel<D, APPEND>), dim3((unsigned)a.Hq, (unsigned)a.B),
                     dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode merge kernel launch");
  return GQA_OK;
}

template <bool APPEND>
int dispatch_decode_part(gqa::DecodeArgs& a, int d, int cus, hipStream_t s) {
  const bool two = a.g > 16;
  switch (d) {
    case 32:
      return two ? launch_decode_part<32, 2, APPEND>(a, cus, s)
                 : launch_decode_part<32, 1, APPEND>(a, cus, s);
    case 64:
      return two ? launch_decode_part<64, 2, APPEND>(a, cus, s)
                 : launch_decode_part<64, 1, APPEND>(a, cus, s);
    default:
      return two ? launch_decode_part<128, 2, APPEND>(a, cus, s)
                 : launch_decode_part<128, 1, APPEND>(a, cus, s);
  }
}

size_t decode_ws_bytes(int B, int Hq, int smax, int d, int split) {
  const size_t ns = (size_t)((smax + split - 1) / split);
  return (size_t)B * Hq * ns * (size_t)(d + 4) * sizeof(float);
}

// Validation and launch arguments of a forward call (everything but the
// schedule): qs / kvs are element strides {batch, head, token} of Q and O /
// of K and V (the head dimension is contiguous); pointers and strides are
// already checked for NULL.  Pure host code: no HIP call.
int fwd_setup(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
              int Nq, int Nk, int d, const int64_t* qs, const int64_t* kvs, int causal,
              int q_offset, float scale, int dtype, gqa::PrefillArgs* out) {
  // ---- validation: host only, before any HIP call
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1)
    return fail(GQA_ERR_BAD_SHAPE, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", B,
                Hq, Hkv, Nq, Nk, d);
  if (causal && q_offset < 0) return fail(GQA_ERR_BAD_SHAPE, "q_offset=%d < 0", q_offset);
  if (Hq % Hkv != 0)
    return fail(GQA_ERR_HEAD_GROUPING, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (!std::isfinite(scale)) return fail(GQA_ERR_UNSUPPORTED, "scale must be finite");
  if ((long long)Nq * d > kIntMax || (long long)Nk * d > kIntMax ||
      (causal && (long long)q_offset + Nq > kIntMax))
    return fail(GQA_ERR_BAD_SHAPE, "sequence too long for 32-bit in-head indexing");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(GQA_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");

  const int M = 32 * kPrefillWaves;
  const int g = Hq / Hkv;
  const int Gu = g < M ? g : M;
  const int R = M / Gu;
  const int HB = (g + Gu - 1) / Gu;
  const long long NQB = ((long long)Nq + R - 1) / R;
  const long long T = (long long)B * Hkv * HB * NQB;
  if (T > kIntMax) return fail(GQA_ERR_BAD_SHAPE, "too many work units (%lld)", T);

  const int esz = dtype == GQA_DTYPE_BF16 ? 2 : 4;
  gqa::PrefillArgs& a = *out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.q_sb = qs[0];
  a.q_sh = qs[1];
  a.q_sn = qs[2];
  a.kv_sb = kvs[0];
  a.kv_sh = kvs[1];
  a.kv_rowb = (int)(kvs[2] * esz);
  a.g = g;
  a.Gu = Gu;
  a.R = R;
  a.HB = HB;
  a.NQB = (int)NQB;
  a.T = (int)T;
  a.q_offset = causal ? q_offset : 0;
  a.c = softmax_coef(scale);
  a.thr = gqa::kRescaleSlack / a.c;
  a.negate_q = scale < 0.f ? 1 : 0;
  return GQA_OK;
}

int fwd_entry(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
              int Nq, int Nk, int d, const int64_t* qs, const int64_t* kvs, int causal,
              int q_offset, float scale, int dtype, void* stream) {
  gqa::PrefillArgs a;
  int st = fwd_setup(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, qs, kvs, causal, q_offset, scale, dtype,
                     &a);
  if (st != GQA_OK) return st;
  int dev = 0;
  DeviceInfo info;
  st = current_device(&dev, &info);
  if (st != GQA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // K/V rows D elements apart: the compile-time stride
  if (kvs[2] == d) {
    if (dtype == GQA_DTYPE_BF16)
      return dispatch_prefill<uint16_t, CfgBf16>(a, d, causal, dev, info, hs);
    return dispatch_prefill<float, CfgF32>(a, d, causal, dev, info, hs);
  }
  if (dtype == GQA_DTYPE_BF16)
    return dispatch_prefill<uint16_t, CfgBf16S>(a, d, causal, dev, info, hs);
  return dispatch_prefill<float, CfgF32S>(a, d, causal, dev, info, hs);
}

// Shared body of the two decode entry points.  knew == NULL: plain decode
// over the cached lengths in lens; otherwise append (lens are positions, the
// caches are written at them).
// Validation and launch arguments of a decode call, all but the split size
// (decode_splits).  Pure host code: no HIP call.
// check_ws == false: the caller supplies the workspace after validation (the
// static scratch of gqa_attn_decode_noalloc, whose size it checks itself).
int decode_setup(const void* q, const void* kcache, const void* vcache, const int32_t* lens,
                 const void* knew, const void* vnew, void* kc_out, void* vc_out, void* o, int B,
                 int Hq, int Hkv, int Smax, int d, float scale, int dtype, void* workspace,
                 size_t workspace_bytes, gqa::DecodeArgs* out, bool check_ws = true,
                 const int32_t* slots = nullptr, int Ncache = 0) {
  const bool append = knew != nullptr;
  if (B < 1 || Hq < 1 || Hkv < 1 || Smax < 1 || d < 1)
    return fail(GQA_ERR_BAD_SHAPE, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Smax=%d d=%d)", B, Hq,
                Hkv, Smax, d);
  if (Hq % Hkv != 0)
    return fail(GQA_ERR_HEAD_GROUPING, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (!std::isfinite(scale)) return fail(GQA_ERR_UNSUPPORTED, "scale must be finite");
  if ((long long)Smax * d > kIntMax)
    return fail(GQA_ERR_BAD_SHAPE, "cache capacity too large for 32-bit in-head indexing");
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o) ||
      (append && (!aligned16(knew) || !aligned16(vnew))))
    return fail(GQA_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  const size_t need = decode_ws_bytes(B, Hq, Smax, d, kMinSplit);
  if (check_ws && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(GQA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const int g = Hq / Hkv;
  const int ncb = (g + 31) / 32;
  if ((long long)Hkv * ncb > 65535 || B > 65535)
    return fail(GQA_ERR_BAD_SHAPE, "grid too large (B=%d, Hkv*blocks=%lld)", B,
                (long long)Hkv * ncb);

  gqa::DecodeArgs& a = *out;
  a.q = q;
  a.kc = kcache;
  a.vc = vcache;
  a.seqlens = lens;
  a.knew = knew;
  a.vnew = vnew;
  a.kc_out = kc_out;
  a.vc_out = vc_out;
  a.o = o;
  a.ws = reinterpret_cast<float*>(workspace);
  a.slots = slots;
  a.Ncache = slots ? Ncache : B;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Smax = Smax;
  a.g = g;
  a.NCB = ncb;
  a.c = softmax_coef(scale);
  a.thr = gqa::kRescaleSlack / a.c;
  a.negate_q = scale < 0.f ? 1 : 0;
  return GQA_OK;
}

void decode_splits(gqa::DecodeArgs& a, int cus, int waves_per_cu = 4) {
  a.S_TOK = decode_split_tokens(a.B, a.Hkv, a.NCB, a.Smax, cus, waves_per_cu);
  a.NS = (a.Smax + a.S_TOK - 1) / a.S_TOK;
}

// static_ws: the records go to this device's static scratch array instead of
// a caller workspace (workspace / workspace_bytes are ignored).
int decode_entry(const void* q, const void* kcache, const void* vcache, const int32_t* lens,
                 const void* knew, const void* vnew, void* kc_out, void* vc_out, void* o, int B,
                 int Hq, int Hkv, int Smax, int d, float scale, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream, bool static_ws = false,
                 const int32_t* slots = nullptr, int Ncache = 0) {
  const bool append = knew != nullptr;
  gqa::DecodeArgs a;
  int st = decode_setup(q, kcache, vcache, lens, knew, vnew, kc_out, vc_out, o, B, Hq, Hkv, Smax,
                        d, scale, dtype, workspace, workspace_bytes, &a, !static_ws, slots,
                        Ncache);
  if (st != GQA_OK) return st;
  if (static_ws) {
    const size_t need = decode_ws_bytes(B, Hq, Smax, d, kMinSplit);
    if (need > kNoAllocScratchBytes)
      return fail(GQA_ERR_WORKSPACE,
                  "this decode needs %zu bytes of split records; the static scratch of "
                  "gqa_attn_decode_noalloc holds %zu",
                  need, kNoAllocScratchBytes);
  }
  int dev = 0;
  DeviceInfo info;
  st = current_device(&dev, &info);
  if (st != GQA_OK) return st;
  if (static_ws) {
    void* p = nullptr;
    st = scratch_address(dev, &p);
    if (st != GQA_OK) return st;
    a.ws = reinterpret_cast<float*>(p);
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == GQA_DTYPE_BF16)
    return append ? dispatch_decode_part<true>(a, d, info.cus, hs)
                  : dispatch_decode_part<false>(a, d, info.cus, hs);
  decode_splits(a, info.cus);
  if (append) return dispatch_decode<float, DecCfgF32, true>(a, d, hs);
  return dispatch_decode<float, DecCfgF32, false>(a, d, hs);
}

// ------------------------------------------------------------------ mixed batch

// One launch over the chunk and the decode work, one workgroup per resident
// slot (fewer if there is less work), then the merge passes.  The chunk runs
// as a prefill call of its shape would run it:
//  * quad units, whose four groups split each 64-column unit's keys, when
//    that call would take them (few, long units);
//  * else, with too few units to balance whole ones, the balanced
//    schedule's pieces (equal key-tile chunks, cut units merged by the
//    prefill merge pass), sized for 1 / kMixedChunkDiv of the resident
//    workgroups, so the others start on the decode work at once instead of
//    waiting for the chunk's few units to end;
//  * else the persistent schedule's 128-column units.
// The decode rows are split as gqa_attn_decode splits them (bf16: the same
// parts, so the same records and bits) and taken by the workgroups that the
// chunk leaves idle.
#ifndef GQA_MIXED_CHUNK_DIV
#define GQA_MIXED_CHUNK_DIV 2
#endif
constexpr int kMixedChunkDiv = GQA_MIXED_CHUNK_DIV;
template <typename T, class C, class CD>
int launch_mixed(gqa::MixedArgs& m, int dev_id, const DeviceInfo& dev, hipStream_t stream) {
  using CQ = gqa::TileCfg<T, C::D, C::BC, 2, C::KVS>;
  enum { kPersistent, kQuad, kBalanced } kind = kPersistent;
  gqa::MixedArgs mq = m;
  if constexpr (8 * CQ::STAGE_BYTES <= kLdsBytes) {
    if (m.p.T > 0) {
      decompose(mq.p, 64);
      const long long t64 = mq.p.T;
      if (m.p.T < dev.cus && 4 * t64 >= 3LL * dev.cus && t64 <= dev.cus &&
          unit_tiles<CQ>(mq.p, true, 0) >= 8)
        kind = kQuad;
    }
  }
  long long cuts = 0;
  const void* bal_kern = reinterpret_cast<const void*>(&gqa::mixed_balanced_kernel<T, C, CD>);
  if (kind != kQuad && m.p.T > 0) {
    const long long chunk_slots =
        std::max(1LL, (long long)dev.cus * occupancy(bal_kern, C::NT) / kMixedChunkDiv);
    if (plan_balanced<C>(m.p, true, chunk_slots, &cuts)) kind = kBalanced;
  }
  gqa::MixedArgs& a = kind == kQuad ? mq : m;
  const void* kern = nullptr;
  int threads = C::NT;
  if constexpr (8 * CQ::STAGE_BYTES <= kLdsBytes) {
    if (kind == kQuad) {
      kern = reinterpret_cast<const void*>(&gqa::mixed_quad_kernel<T, CQ, CD>);
      threads = 4 * CQ::NT;
    }
  }
  if (kind == kBalanced) kern = bal_kern;
  if (kind == kPersistent) kern = reinterpret_cast<const void*>(&gqa::mixed_kernel<T, C, CD>);
  const long long slots = (long long)dev.cus * occupancy(kern, threads);
  constexpr bool REG = !std::is_same<T, float>::value;
  int dw = 1;
  if constexpr (REG) {  // bf16: each group of W waves takes a decode part
    dw = (threads / 64) / (m.d.g > 16 ? PartCfgOf<C::D, 2>::W : PartCfgOf<C::D, 1>::W);
  } else {
    dw = gqa::mixed_decode_waves<C, CD>();
    if constexpr (8 * CQ::STAGE_BYTES <= kLdsBytes) {
      if (kind == kQuad) dw = gqa::mixed_quad_decode_waves<CQ, CD>();
    }
  }
  if (a.d.B > 0) {
    if constexpr (REG) {
      // bf16: the parts of gqa_attn_decode (the same records, and outputs)
      if (a.d.g > 16) part_plan<PartCfgOf<C::D, 2>>(a.d, dev.cus);
      else part_plan<PartCfgOf<C::D, 1>>(a.d, dev.cus);
    } else {
      decode_splits(a.d, dev.cus, a.p.T >= slots ? 8 : 4);
    }
    const long long nd = (long long)a.d.NS * a.d.Hkv * a.d.NCB * a.d.B;
    if (nd > kIntMax / 2) return fail(GQA_ERR_BAD_SHAPE, "too many decode splits (%lld)", nd);
    a.nd = (int)nd;
  }
  const long long pieces = kind == kBalanced ? (long long)a.p.nsl * a.p.Pp : 0;
  const long long items = kind == kBalanced ? pieces : a.p.T;
  const long long work = items + ((long long)a.nd + dw - 1) / dw;
  const long long grid = std::max<long long>(
      std::max<long long>(1, pieces), std::min<long long>(work, slots));
  const size_t ws_bytes =
      cuts > 0 ? (size_t)pieces * 2 * gqa::part_floats<C>() * sizeof(float) : 0;
  StreamState ss;
  int st = stream_state(dev_id, stream, ws_bytes, &ss);
  if (st != GQA_OK) return st;
  a.p.ctr = ss.ctr;
  a.p.zero = 0;
  a.p.ws = cuts > 0 ? ss.ws : nullptr;
  (void)hipGetLastError();  // a stale error belongs to an earlier call
  if constexpr (8 * CQ::STAGE_BYTES <= kLdsBytes) {
    if (kind == kQuad)
      hipLaunchKernelGGL((gqa::mixed_quad_kernel<T, CQ, CD>), dim3((unsigned)grid),
                         dim3(4 * CQ::NT), 0, stream, a);
  }
  if (kind == kBalanced)
    hipLaunchKernelGGL((gqa::mixed_balanced_kernel<T, C, CD>), dim3((unsigned)grid), dim3(C::NT),
                       0, stream, a);
  if (kind == kPersistent)
    hipLaunchKernelGGL((gqa::mixed_kernel<T, C, CD>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "mixed kernel launch");
  if (cuts > 0) {
    hipLaunchKernelGGL((gqa::prefill_merge_kernel<T, C, true>),
                       dim3((unsigned)(a.p.nsl * (a.p.Pp - 1) * C::NW)), dim3(64 * C::DB), 0,
                       stream, a.p);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "prefill merge kernel launch");
  }
  if (a.nd > 0) {
    if constexpr (REG)
      hipLaunchKernelGGL((gqa::decode_merge_kernel<C::D, false>),
                         dim3((unsigned)a.d.Hq, (unsigned)a.d.B), dim3(256), 0, stream, a.d);
    else
      hipLaunchKernelGGL((gqa::decode_combine_kernel<T, C::D, false>),
                         dim3((unsigned)a.d.Hq, (unsigned)a.d.B), dim3(256), 0, stream, a.d);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "decode combine kernel launch");
  }
  return GQA_OK;
}

template <typename T, template <int> class Cfg, template <int> class DCfg>
int dispatch_mixed(gqa::MixedArgs& m, int d, int dev_id, const DeviceInfo& dev,
                   hipStream_t s) {
  switch (d) {
    case 32: return launch_mixed<T, Cfg<32>, DCfg<32>>(m, dev_id, dev, s);
    case 64: return launch_mixed<T, Cfg<64>, DCfg<64>>(m, dev_id, dev, s);
    default: return launch_mixed<T, Cfg<128>, DCfg<128>>(m, dev_id, dev, s);
  }
}

int mixed_entry(const void* q, const void* k, const void* v, void* o, int B, int Nq, int Nk,
                int q_offset, const void* qd, const void* kcache, const void* vcache,
                const int32_t* seqlens, void* od, int Bd, int Smax, int Hq, int Hkv, int d,
                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  // ---- validation: host only, before any HIP call
  if (B < 0 || Bd < 0)
    return fail(GQA_ERR_BAD_SHAPE, "part sizes must be >= 0 (B=%d Bd=%d)", B, Bd);
  if (B > 0 && (!q || !k || !v || !o))
    return fail(GQA_ERR_NULL_POINTER, "q, k, v and o must be non-NULL when B > 0");
  if (Bd > 0 && (!qd || !kcache || !vcache || !seqlens || !od))
    return fail(GQA_ERR_NULL_POINTER,
                "qd, kcache, vcache, seqlens and od must be non-NULL when Bd > 0");
  gqa::MixedArgs m;
  std::memset(&m, 0, sizeof(m));
  if (B > 0) {
    // contiguous strides, computed only from sizes whose products fit; any
    // other size is rejected by fwd_setup's own checks
    const bool fits = Hq >= 1 && Hkv >= 1 && Nq >= 1 && Nk >= 1 && d >= 1 &&
                      (long long)Nq * d <= kIntMax && (long long)Nk * d <= kIntMax;
    const int64_t qs[3] = {fits ? (int64_t)Hq * Nq * d : 0, fits ? (int64_t)Nq * d : 0, d};
    const int64_t kvs[3] = {fits ? (int64_t)Hkv * Nk * d : 0, fits ? (int64_t)Nk * d : 0, d};
    if (fits && (qs[0] > (1LL << 62) / B || kvs[0] > (1LL << 62) / B))
      return fail(GQA_ERR_BAD_SHAPE, "chunk tensors too large");
    int st = fwd_setup(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, qs, kvs, 1, q_offset, scale, dtype,
                       &m.p);
    if (st != GQA_OK) return st;
  } else {
    m.p.Hkv = 1;  // no units: every prefill queue is empty
    m.p.HB = 1;
    m.p.NQB = 1;
  }
  if (Bd > 0) {
    int st = decode_setup(qd, kcache, vcache, seqlens, nullptr, nullptr, nullptr, nullptr, od, Bd,
                          Hq, Hkv, Smax, d, scale, dtype, workspace, workspace_bytes, &m.d);
    if (st != GQA_OK) return st;
  }
  if (B == 0 && Bd == 0) return GQA_OK;  // nothing to compute

  // ---- device
  int dev = 0;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != GQA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (dtype == GQA_DTYPE_BF16)
    return dispatch_mixed<uint16_t, CfgBf16, DecCfgBf16>(m, d, dev, info, hs);
  return dispatch_mixed<float, CfgF32, DecCfgF32>(m, d, dev, info, hs);
}

// ------------------------------------------------------------------ backward

// Query parts per dK/dV key block (64 keys): about four dK/dV workgroups
// per CU of a 256-CU gfx950 part, at most kBwdQuerySplitMax.  The kernels
// take their blocks heaviest key block first, so a causal launch balances
// with a few rounds of workgroups; more parts only add records for the
// merge to read.  A function of the shape alone, so that the workspace
// query and the launch agree.
constexpr long long kBwdSplitBlocks = 4LL * 256;
int bwd_query_parts(int B, int Hkv, int Nk) {
  const long long blocks = (long long)((Nk + 63) / 64) * Hkv * B;
  const long long qs = (kBwdSplitBlocks + blocks - 1) / blocks;
  return (int)std::max(1LL, std::min<long long>(qs, gqa::kBwdQuerySplitMax));
}

// Backward workspace: the row statistics (log-sum-exp, D: 2 fp32 per query
// row, rounded up to 16 bytes), then, with more than one query part, the
// parts' fp32 dK, dV records.
size_t bwd_stats_bytes(int B, int Hq, int Nq) {
  return (2 * (size_t)B * Hq * Nq * sizeof(float) + 15) / 16 * 16;
}
size_t bwd_ws_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  const int qs = bwd_query_parts(B, Hkv, Nk);
  return bwd_stats_bytes(B, Hq, Nq) +
         (qs > 1 ? (size_t)qs * 2 * B * Hkv * Nk * d * sizeof(float) : 0);
}

template <typename T, class C, bool CAUSAL>
int launch_bwd(gqa::BwdArgs& ba, hipStream_t stream) {
  (void)hipGetLastError();  // a stale error belongs to an earlier call
  hipLaunchKernelGGL((gqa::bwd_dq_kernel<T, C, CAUSAL>), dim3((unsigned)ba.f.T), dim3(C::NT), 0,
                     stream, ba);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "backward dQ kernel launch");
  // dK/dV: 64 keys per workgroup, so that the LLaMA-sized launches spread
  // over every CU: bf16 at d = 128 as four 16-key waves on the 16x16x32
  // MFMA (two waves per SIMD), otherwise two 32-key waves (their registers
  // allow one wave per SIMD)
  using CK = gqa::TileCfg<T, C::D, C::BC, 2>;
  const unsigned kblocks = (unsigned)((ba.f.Nk + 32 * CK::NW - 1) / (32 * CK::NW));
  ba.qsplit = bwd_query_parts(ba.f.B, ba.f.Hkv, ba.f.Nk);
  const dim3 kgrid(kblocks * (unsigned)ba.qsplit, (unsigned)ba.f.Hkv, (unsigned)ba.f.B);
  if constexpr (std::is_same<T, uint16_t>::value && C::D == 128) {
    using C16 = gqa::TileCfg<T, C::D, 32, 4>;
    hipLaunchKernelGGL((gqa::bwd_dkdv16_kernel<C16, CAUSAL>), kgrid, dim3(C16::NT), 0, stream,
                       ba);
  } else {
    hipLaunchKernelGGL((gqa::bwd_dkdv_kernel<T, CK, CAUSAL>), kgrid, dim3(CK::NT), 0, stream,
                       ba);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "backward dK/dV kernel launch");
  if (ba.qsplit == 1) return GQA_OK;
  const long long n4 = 2LL * ba.f.B * ba.f.Hkv * ba.f.Nk * C::D / 4;
  long long mblocks = (n4 + 255) / 256;
  if (mblocks > 4096) mblocks = 4096;
  hipLaunchKernelGGL((gqa::bwd_merge_kernel<T>), dim3((unsigned)mblocks), dim3(256), 0, stream,
                     ba, n4);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "backward dK/dV merge kernel launch");
  return GQA_OK;
}

template <typename T, template <int> class Cfg>
int dispatch_bwd(gqa::BwdArgs& ba, int d, int causal, hipStream_t s) {
  switch (d) {
    case 32: return causal ? launch_bwd<T, Cfg<32>, true>(ba, s) : launch_bwd<T, Cfg<32>, false>(ba, s);
    case 64: return causal ? launch_bwd<T, Cfg<64>, true>(ba, s) : launch_bwd<T, Cfg<64>, false>(ba, s);
    default:
      return causal ? launch_bwd<T, Cfg<128>, true>(ba, s) : launch_bwd<T, Cfg<128>, false>(ba, s);
  }
}

int bwd_entry(const void* q, const void* k, const void* v, const void* o, const void* dout,
              void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
              int causal, int q_offset, float scale, int dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1)
    return fail(GQA_ERR_BAD_SHAPE, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d)", B,
                Hq, Hkv, Nq, Nk, d);
  if (causal && q_offset < 0) return fail(GQA_ERR_BAD_SHAPE, "q_offset=%d < 0", q_offset);
  if (Hq % Hkv != 0)
    return fail(GQA_ERR_HEAD_GROUPING, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GQA_ERR_UNSUPPORTED, "the backward needs a finite scale > 0");
  if ((long long)Nq * d > kIntMax || (long long)Nk * d > kIntMax ||
      (causal && (long long)q_offset + Nq > kIntMax))
    return fail(GQA_ERR_BAD_SHAPE, "sequence too long for 32-bit in-head indexing");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(GQA_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  const size_t need = bwd_ws_bytes(B, Hq, Hkv, Nq, Nk, d);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(GQA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const int M = 32 * kPrefillWaves;
  const int g = Hq / Hkv;
  const int Gu = g < M ? g : M;
  const int R = M / Gu;
  const long long NQB = ((long long)Nq + R - 1) / R;
  const long long T = (long long)B * Hkv * ((g + Gu - 1) / Gu) * NQB;
  if (T > kIntMax || B > 65535 || Hkv > 65535)
    return fail(GQA_ERR_BAD_SHAPE, "too many work units (%lld)", T);
  // the row statistics are addressed with 32-bit byte offsets
  if (8LL * B * Hq * Nq > 4294967295LL)
    return fail(GQA_ERR_BAD_SHAPE, "too many query rows (%lld)", (long long)B * Hq * Nq);

  int dev = 0;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != GQA_OK) return st;

  const int esz = dtype == GQA_DTYPE_BF16 ? 2 : 4;
  gqa::BwdArgs ba;
  gqa::PrefillArgs& a = ba.f;
  a = gqa::PrefillArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.q_sb = (long long)Hq * Nq * d;
  a.q_sh = (long long)Nq * d;
  a.q_sn = d;
  a.kv_sb = (long long)Hkv * Nk * d;
  a.kv_sh = (long long)Nk * d;
  a.kv_rowb = d * esz;
  a.g = g;
  decompose(a, M);
  a.q_offset = causal ? q_offset : 0;
  a.c = scale * gqa::kLog2e;
  a.thr = gqa::kRescaleSlack / a.c;
  ba.o = o;
  ba.dout = dout;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.lse = reinterpret_cast<float*>(workspace);
  ba.dd = ba.lse + (size_t)B * Hq * Nq;
  ba.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                     bwd_stats_bytes(B, Hq, Nq));
  ba.scale = scale;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (dtype == GQA_DTYPE_BF16) return dispatch_bwd<uint16_t, CfgBf16>(ba, d, causal, hs);
  return dispatch_bwd<float, CfgF32>(ba, d, causal, hs);
}

}  // namespace

extern "C" {

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL_POINTER: return "null pointer";
    case GQA_ERR_BAD_SHAPE: return "bad shape";
    case GQA_ERR_HEAD_GROUPING: return "query heads not a multiple of key/value heads";
    case GQA_ERR_UNSUPPORTED: return "unsupported argument";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_NO_DEVICE: return "no gfx950 device";
    case GQA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* gqa_last_error_string(void) { return g_last_error.c_str(); }

int gqa_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d, int causal, int q_offset, float scale, int dtype,
                 void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o) return fail(GQA_ERR_NULL_POINTER, "q, k, v and o must be non-NULL");
  // contiguous [B, H, N, d]
  const int64_t qs[3] = {(int64_t)Hq * Nq * d, (int64_t)Nq * d, (int64_t)d};
  const int64_t kvs[3] = {(int64_t)Hkv * Nk * d, (int64_t)Nk * d, (int64_t)d};
  return fwd_entry(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, qs, kvs, causal, q_offset, scale, dtype,
                   stream);
}

int gqa_attn_fwd_strided(const void* q, const void* k, const void* v, void* o, int B, int Hq,
                         int Hkv, int Nq, int Nk, int d, const int64_t* q_strides,
                         const int64_t* kv_strides, int causal, int q_offset, float scale,
                         int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !q_strides || !kv_strides)
    return fail(GQA_ERR_NULL_POINTER, "q, k, v, o, q_strides and kv_strides must be non-NULL");
  for (int i = 0; i < 3; ++i)
    if (q_strides[i] < 0 || kv_strides[i] < 0)
      return fail(GQA_ERR_BAD_SHAPE, "strides must be >= 0");
  const int64_t esz = dtype == GQA_DTYPE_BF16 ? 2 : 4;
  for (int i = 0; i < 3; ++i)
    if ((q_strides[i] * esz) % 16 != 0 || (kv_strides[i] * esz) % 16 != 0)
      return fail(GQA_ERR_UNSUPPORTED, "strides must be multiples of 16 bytes");
  // O is written through the Q strides: its rows must not overlap.  Sorted by
  // stride, every dimension of extent > 1 must step past the whole extent of
  // the ones inside it (the head dimension, stride 1, innermost).
  if (B >= 1 && Hq >= 1 && Nq >= 1 && d >= 1) {
    int64_t st[3] = {q_strides[0], q_strides[1], q_strides[2]};
    int64_t ex[3] = {B, Hq, Nq};
    for (int x = 0; x < 3; ++x)
      for (int y = x + 1; y < 3; ++y)
        if (st[y] < st[x]) {
          std::swap(st[x], st[y]);
          std::swap(ex[x], ex[y]);
        }
    int64_t span = d;  // elements covered by the dimensions inside
    for (int x = 0; x < 3; ++x) {
      if (ex[x] == 1) continue;
      if (st[x] < span)
        return fail(GQA_ERR_BAD_SHAPE, "q/o strides make output rows overlap");
      span = st[x] * ex[x];
    }
  }
  if (kv_strides[2] * esz * 64 > kIntMax)
    return fail(GQA_ERR_BAD_SHAPE, "k/v token stride too large (%lld elements)",
                (long long)kv_strides[2]);
  return fwd_entry(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, q_strides, kv_strides, causal, q_offset,
                   scale, dtype, stream);
}

int gqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                        int max_seqlen_q, int Hq, int Hkv, int d, int causal, float scale,
                        int dtype, void* stream) {
  g_last_error.clear();
  return varlen_entry(q, k, v, o, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, Hq, Hkv, d,
                      causal, scale, dtype, stream);
}

size_t gqa_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Smax, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Smax < 1 || !head_dim_ok(d) || Hq % Hkv != 0) return 0;
  return decode_ws_bytes(B, Hq, Smax, d, kMinSplit);
}

int gqa_attn_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int Smax, int d,
                    float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error.clear();
  if (!q || !kcache || !vcache || !seqlens || !o)
    return fail(GQA_ERR_NULL_POINTER, "q, kcache, vcache, seqlens and o must be non-NULL");
  return decode_entry(q, kcache, vcache, seqlens, nullptr, nullptr, nullptr, nullptr, o, B, Hq,
                      Hkv, Smax, d, scale, dtype, workspace, workspace_bytes, stream);
}

int gqa_attn_decode_append(const void* q, const void* k_new, const void* v_new, void* kcache,
                           void* vcache, const int32_t* positions, void* o, int B, int Hq,
                           int Hkv, int Smax, int d, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k_new || !v_new || !kcache || !vcache || !positions || !o)
    return fail(GQA_ERR_NULL_POINTER,
                "q, k_new, v_new, kcache, vcache, positions and o must be non-NULL");
  return decode_entry(q, kcache, vcache, positions, k_new, v_new, kcache, vcache, o, B, Hq, Hkv,
                      Smax, d, scale, dtype, workspace, workspace_bytes, stream);
}

int gqa_attn_decode_slots(const void* q, const void* k_new, const void* v_new, void* kcache,
                          void* vcache, int Ncache, const int32_t* slots, const int32_t* lengths,
                          void* o, int B, int Hq, int Hkv, int Smax, int d, float scale,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !kcache || !vcache || !slots || !lengths || !o)
    return fail(GQA_ERR_NULL_POINTER, "q, kcache, vcache, slots, lengths and o must be non-NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(GQA_ERR_NULL_POINTER, "k_new and v_new must both be given or both be NULL");
  if (Ncache < 1) return fail(GQA_ERR_BAD_SHAPE, "Ncache must be >= 1 (got %d)", Ncache);
  const bool append = k_new != nullptr;
  return decode_entry(q, kcache, vcache, lengths, k_new, v_new, append ? kcache : nullptr,
                      append ? vcache : nullptr, o, B, Hq, Hkv, Smax, d, scale, dtype, workspace,
                      workspace_bytes, stream, false, slots, Ncache);
}

int gqa_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* seqlens, void* o, int B, int Hq, int Hkv, int Smax,
                            int d, float scale, int dtype, void* stream) {
  g_last_error.clear();
  if (!q || !kcache || !vcache || !seqlens || !o)
    return fail(GQA_ERR_NULL_POINTER, "q, kcache, vcache, seqlens and o must be non-NULL");
  return decode_entry(q, kcache, vcache, seqlens, nullptr, nullptr, nullptr, nullptr, o, B, Hq,
                      Hkv, Smax, d, scale, dtype, nullptr, 0, stream, true);
}

size_t gqa_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || !head_dim_ok(d) || Hq % Hkv != 0)
    return 0;
  return bwd_ws_bytes(B, Hq, Hkv, Nq, Nk, d);
}

int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 int causal, int q_offset, float scale, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !dout || !dq || !dk || !dv)
    return fail(GQA_ERR_NULL_POINTER, "q, k, v, o, dout, dq, dk and dv must be non-NULL");
  return bwd_entry(q, k, v, o, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, scale,
                   dtype, workspace, workspace_bytes, stream);
}

int gqa_attn_mixed(const void* q, const void* k, const void* v, void* o, int B, int Nq, int Nk,
                   int q_offset, const void* qd, const void* kcache, const void* vcache,
                   const int32_t* seqlens, void* od, int Bd, int Smax, int Hq, int Hkv, int d,
                   float scale, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  g_last_error.clear();
  return mixed_entry(q, k, v, o, B, Nq, Nk, q_offset, qd, kcache, vcache, seqlens, od, Bd, Smax,
                     Hq, Hkv, d, scale, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
