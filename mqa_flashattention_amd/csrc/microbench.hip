// microbench.hip -- machine-peak microbenchmarks (libgqa_microbench.so).
//
// Measurement infrastructure for bench.py, not part of the attention path:
// it puts the attention kernels' throughput beside what the MI355X in hand
// actually sustains, next to the published peaks.
//   * gqa_mb_mfma_bf16: dense v_mfma_f32_32x32x16_bf16 issue rate, four
//     independent accumulators per wave, operands in registers (no memory
//     traffic), two waves per SIMD;
//   * gqa_mb_read: streaming read of a device buffer with 16-byte loads
//     (the HBM read rate once the buffer exceeds the 256 MB Infinity Cache);
//   * the shader clock under MFMA load: wave 0 of the MFMA kernel reads the
//     core-clock counter (s_memtime) and the constant 100 MHz counter
//     (s_memrealtime) at its start and end;
//   * gqa_mb_lds: LDS access patterns of the attention kernels' tile reads
//     and staging writes, each repeated by every wave; the time per pattern
//     over the linear pattern's of the same width is its bank-conflict
//     factor (rocprofv3's SQ_LDS_BANK_CONFLICT over SQ_INSTS_LDS gives the
//     same answer in conflict cycles);
//   * gqa_mb_valu: the vector-ALU rate of the two operations the softmax
//     spends its time on, fp32 FMA and the hardware exp2 (v_exp_f32), each
//     as eight independent chains per lane, with wave 0's clock counters
//     as in the MFMA kernel.
// Each call is asynchronous on the given stream; the caller times it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, unsigned long long* clk,
                                                        float* sink) {
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 5);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  // never true for these operands; keeps the MFMAs alive
  if (s == -1.0f) sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (timer) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

__global__ void __launch_bounds__(256) read_peak_kernel(const u32x4* __restrict__ p, size_t n,
                                                        uint32_t* sink) {
  u32x4 x = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // eight 16-byte loads in flight per thread
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  for (; i < n; i += stride) x ^= p[i];
  // never true for a zero-filled buffer; keeps the loads alive
  if ((x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x9e3779b9u) sink[threadIdx.x] = x[0];
}

// Byte address of lane `lane`'s access in step k of LDS pattern pat, inside
// one wave's 16 KiB window (every pattern stays below 16 KiB).
__device__ __forceinline__ int lds_addr(int pat, int lane, int k) {
  const int n = lane & 15, G = lane >> 4;   // 16-lane groups (the 16x16x32 MFMA's layout)
  const int j = lane & 31, h2 = lane >> 5;  // half-waves (the 32x32x16 MFMA's layout)
  switch (pat) {
    case 0:  // 16-byte reads, linear
      return lane * 16;
    case 1: {  // forward K fragments: row k_row_perm(j) of 272-byte rows, chunk 2 k + h2
      const int r = (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
      return r * 272 + 16 * (2 * (k & 7) + h2);
    }
    case 2:  // forward V^T fragments: 32 consecutive 80-byte rows, columns 32 hk + 16 h2
      return (32 * (k & 3) + j) * 80 + 32 * ((k >> 2) & 1) + 16 * h2;
    case 3:  // dK/dV score operands: rows 8 (n / 4) + 4 qb + n % 4 of 272-byte rows
      return (8 * (n >> 2) + 4 * (k & 1) + (n & 3)) * 272 + 16 * G + 64 * ((k >> 1) & 3);
    case 4:  // dK/dV transposed operands: 16 consecutive 80-byte rows
      return (16 * (k & 7) + n) * 80 + 16 * G;
    case 5: {  // the score operands of case 3 from 256-byte rows, row 16 qb + n, chunk ^ row
      const int c = G + 4 * ((k >> 1) & 3);
      return (16 * (k & 1) + n) * 256 + ((c ^ n) << 4);
    }
    case 6:  // the transposed operands of case 4 from 96-byte rows
      return (16 * (k & 7) + n) * 96 + 16 * G;
    case 7:  // 4-byte writes, linear
      return lane * 4;
    case 8:  // transposed staging writes: two-key words into 80-byte rows
      return (G * 8 + (k & 7)) * 80 + n * 4;
    case 9:  // 16-byte writes, linear
      return lane * 16;
    case 10:  // row-major staging writes: rows 2 n + i of 272-byte rows, chunk G
      return (2 * n + (k & 1)) * 272 + G * 16;
  }
  return 0;
}

// Patterns 0-6 are 16-byte reads, 7-8 4-byte writes, 9-10 16-byte writes.
constexpr int kLdsPatterns = 11;

template <int KIND>  // 0: 16-byte read, 1: 4-byte write, 2: 16-byte write
__global__ void __launch_bounds__(256) lds_pattern_kernel(int pat, int reps, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int lane = threadIdx.x & 63;
  const int base = (threadIdx.x >> 6) * 16384;  // each wave in its own window
  for (int i = threadIdx.x; i < 65536 / 16; i += 256)
    reinterpret_cast<u32x4*>(lds)[i] = u32x4{1u, 2u, 3u, 4u};
  __syncthreads();
  uint32_t acc = 0;
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int a = base + lds_addr(pat, lane, k);
      if constexpr (KIND == 0) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + a);
        acc += v[0] ^ v[3];
      } else if constexpr (KIND == 1) {
        *reinterpret_cast<uint32_t*>(lds + a) = acc + k;
      } else {
        *reinterpret_cast<u32x4*>(lds + a) = u32x4{acc, (uint32_t)k, 0u, 0u};
      }
    }
    __builtin_amdgcn_s_barrier();
  }
  __syncthreads();
  // never true for these values; keeps the accesses alive
  if ((acc ^ reinterpret_cast<const uint32_t*>(lds)[threadIdx.x]) == 0x9e3779b9u)
    sink[threadIdx.x] = acc;
}

template <int OP>  // 0: fp32 FMA, 1: exp2
__global__ void __launch_bounds__(256) valu_rate_kernel(int iters, unsigned long long* clk,
                                                        float* sink) {
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = -0.001f * (float)((threadIdx.x + c) & 15);
  const float a = 0.999f, b = -0.0001f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (OP == 0)
        x[c] = __builtin_fmaf(x[c], a, b);
      else
        x[c] = __builtin_amdgcn_exp2f(x[c]) - 1.0f;  // stays in (-1, 0]: no overflow
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += x[c];
  // never true for these values; keeps the chains alive
  if (sum == 12345.0f) sink[blockIdx.x * 256 + threadIdx.x] = sum;
  if (timer) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// op 0: fp32 FMA, 1: exp2 (plus one subtraction per exp); blocks of 256
// threads, iters x 8 operations per lane.  clk_out (device, 2 x u64) as in
// gqa_mb_mfma_bf16; sink: blocks x 256 floats (device).
int gqa_mb_valu(int op, int blocks, int iters, unsigned long long* clk_out, float* sink,
                void* stream) {
  if (op < 0 || op > 1 || blocks < 1 || iters < 1 || !clk_out || !sink) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (op == 0)
    hipLaunchKernelGGL(valu_rate_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, iters, clk_out, sink);
  else
    hipLaunchKernelGGL(valu_rate_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, iters, clk_out, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// LDS pattern pat (0 .. 10: see lds_addr), blocks of 256 threads, reps x 16
// accesses per wave; sink: 256 uint32 (device).
int gqa_mb_lds(int pat, int blocks, int reps, uint32_t* sink, void* stream) {
  if (pat < 0 || pat >= kLdsPatterns || blocks < 1 || reps < 1 || !sink) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (pat <= 6)
    hipLaunchKernelGGL(lds_pattern_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, pat, reps, sink);
  else if (pat <= 8)
    hipLaunchKernelGGL(lds_pattern_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, pat, reps, sink);
  else
    hipLaunchKernelGGL(lds_pattern_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, pat, reps, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// blocks of 256 threads, iters x 4 MFMAs per wave (32768 FLOPs each).
// clk_out (device, 2 x u64): core-clock and 100 MHz counter deltas of wave 0.
int gqa_mb_mfma_bf16(int blocks, int iters, unsigned long long* clk_out, float* sink,
                     void* stream) {
  if (blocks < 1 || iters < 1 || !clk_out || !sink) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, clk_out, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads bytes (a multiple of 16) of buf once; sink: 256 uint32 (device).
int gqa_mb_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % 16 != 0) return 1;
  hipLaunchKernelGGL(read_peak_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
