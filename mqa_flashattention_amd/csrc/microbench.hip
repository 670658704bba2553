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
//     (s_memrealtime) at its start and end.
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

}  // namespace

extern "C" {

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
