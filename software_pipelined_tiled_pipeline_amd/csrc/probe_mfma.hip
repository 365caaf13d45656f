// Measurement aid, not part of the GEMM path: the rate v_mfma_f32_16x16x32_f16
// (the GEMM's instruction) sustains on this device with no memory traffic at
// all, and the shader clock it runs at.  Every wave keeps the GEMM's 8 x 8
// accumulator tiles (in AGPRs, tied to the instruction as in the GEMM) and
// two sets of operand fragments, and alternates between the sets, so the
// operand bits change every 64 MFMAs as they do in a GEMM.  With random
// operands the chip runs it at the clock its power limit allows; with zero
// operands it shows the issue-bound rate.  A GEMM also spends power on data
// movement and loses issue slots to it, so this loop is a reference point,
// not an upper bound that a GEMM could not pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgemm_probe.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGrid = 1024, kThreads = 256, kBlocks = 8;

// binary16 bits of a value uniform in [-1, 1): SplitMix64 of the index
// (Steele, Lea & Flood 2014), top 53 bits as a fraction, rounded by the
// hardware conversion.
__device__ uint32_t operand_bits(uint64_t i) {
  uint64_t z = i * 0x9E3779B97F4A7C15ull + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  const float u = (float)((double)(z >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
  const _Float16 h = (_Float16)u;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ u32x4 fragment(int zero, uint64_t base) {
  u32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v[k] = zero ? 0u : (operand_bits(base + 2 * k) | (operand_bits(base + 2 * k + 1) << 16));
  return v;
}

__device__ __forceinline__ void mfma(u32x4 a, u32x4 b, f32x4 &c) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

__global__ void __launch_bounds__(kThreads, 1) mfma_loop(int zero, int iters, float *sink, uint64_t *clocks) {
  const uint64_t lane = threadIdx.x & 63;
  u32x4 a[2][kBlocks], b[2][kBlocks];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < kBlocks; ++r) {
      a[s][r] = fragment(zero, ((uint64_t)(s * 2 * kBlocks + r) * 64 + lane) * 8);
      b[s][r] = fragment(zero, ((uint64_t)(s * 2 * kBlocks + kBlocks + r) * 64 + lane) * 8);
    }
  f32x4 acc[kBlocks][kBlocks];
#pragma unroll
  for (int i = 0; i < kBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
      asm volatile("" : "+a"(acc[i][j]));
    }
  asm volatile("s_nop 4");  // accumulator writes -> MFMA srcC
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < kBlocks; ++i)
#pragma unroll
        for (int j = 0; j < kBlocks; ++j) mfma(b[s][j], a[s][i], acc[i][j]);
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // last MFMA -> reads of its result
#pragma unroll
  for (int i = 0; i < kBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) asm volatile("" : "+a"(acc[i][j]));
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clocks[0] = t1 - t0;  // shader clock cycles
    clocks[1] = r1 - r0;  // 100 MHz reference ticks
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kBlocks; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += acc[i][j][r];
  sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int pgemm_probe_mfma(int zero_operands, int64_t iters, double *tflops, double *sclk_ghz) {
  if (!tflops || !sclk_ghz || iters <= 0 || iters > (1 << 24)) return 1;
  float *sink = nullptr;
  uint64_t *clocks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 2;
  uint64_t c[2] = {0, 0};
  float ms = 0.0f;
  if (hipMalloc(&sink, sizeof(float) * kGrid * kThreads) != hipSuccess) goto done;
  if (hipMalloc(&clocks, 2 * sizeof(uint64_t)) != hipSuccess) goto done;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  hipLaunchKernelGGL(mfma_loop, dim3(kGrid), dim3(kThreads), 0, nullptr, zero_operands, (int)iters, sink, clocks);
  if (hipEventRecord(e0, nullptr) != hipSuccess) goto done;
  hipLaunchKernelGGL(mfma_loop, dim3(kGrid), dim3(kThreads), 0, nullptr, zero_operands, (int)iters, sink, clocks);
  if (hipEventRecord(e1, nullptr) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.0f) goto done;
  if (hipMemcpy(c, clocks, sizeof c, hipMemcpyDeviceToHost) != hipSuccess || c[1] == 0) goto done;
  // 4 waves x iters x 2 sets x 64 MFMAs x 16x16x32x2 flop per workgroup
  *tflops = (double)kGrid * 4 * (double)iters * 2 * kBlocks * kBlocks * 16384.0 / (ms * 1e-3) / 1e12;
  *sclk_ghz = (double)c[0] / ((double)c[1] * 10.0);
  rc = 0;
done:
  if (rc) (void)hipGetLastError();
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (clocks) (void)hipFree(clocks);
  return rc;
}
