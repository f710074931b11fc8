// ns_peak.hip - calibration of the matrix-core roofline on the running GPU.
//
// A register-only MFMA loop: every wave issues back-to-back MFMAs on four
// independent accumulators, with operands that change from one instruction
// to the next (random bf16 / fp32 bit patterns, so the multipliers toggle as
// they do on real data).  Nothing is read from memory inside the loop, so
// the achieved rate is what the matrix cores deliver at the clock the chip
// holds under that load.  Each workgroup also reads the shader clock counter
// (s_memtime) and the constant-rate wall clock (s_memrealtime) around its
// loop, which gives the average shader clock during the run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ns_kernels.h"

namespace ns {

namespace {

typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pk_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPeakAcc = 4;  // independent accumulators per wave

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// a bf16 pair with random signs and mantissas, exponents near 1 (|v| in [0.5, 2))
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  const uint32_t lo = (h & 0x807fu) | 0x3f00u, hi = ((h >> 16) & 0x807fu) | 0x3f00u;
  return lo | (hi << 16);
}

template <int DT>  // 1: bf16 32x32x16, 0: fp32 32x32x2
__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(float* sink, unsigned long long* clocks,
                                                                  int iters) {
  const uint32_t tid = blockIdx.x * kPeakThreads + threadIdx.x;
  pk_f32x16 acc[kPeakAcc];
#pragma unroll
  for (int a = 0; a < kPeakAcc; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[a][r] = 0.0f;
  // four A and four B operand registers per lane
  uint4 A[4], B[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t s = mix32(tid * 8u + (uint32_t)j);
    A[j] = make_uint4(rand_bf16x2(mix32(s + 1)), rand_bf16x2(mix32(s + 2)), rand_bf16x2(mix32(s + 3)),
                      rand_bf16x2(mix32(s + 4)));
    B[j] = make_uint4(rand_bf16x2(mix32(s + 5)), rand_bf16x2(mix32(s + 6)), rand_bf16x2(mix32(s + 7)),
                      rand_bf16x2(mix32(s + 8)));
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int a = 0; a < kPeakAcc; ++a) {
        const uint4 x = A[a], y = B[(a + u) & 3];
        if constexpr (DT == 1) {
          acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pk_bf16x8, x),
                                                           __builtin_bit_cast(pk_bf16x8, y), acc[a], 0, 0, 0);
        } else {
          acc[a] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(x.x), __uint_as_float(y.x), acc[a], 0, 0, 0);
        }
      }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < kPeakAcc; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[a][r];
  sink[tid] = s;  // keeps every product live
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

}  // namespace

hipError_t launch_mfma_peak(int dtype, int blocks, int iters, float* sink, unsigned long long* clocks,
                            hipStream_t st) {
  if (dtype == 1)
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(kPeakThreads), 0, st, sink, clocks, iters);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(kPeakThreads), 0, st, sink, clocks, iters);
  return hipGetLastError();
}

// FLOPs of one wave's MFMA instruction of the peak loop
long long mfma_peak_flops_per_inst(int dtype) { return dtype == 1 ? 2LL * 32 * 32 * 16 : 2LL * 32 * 32 * 2; }
int mfma_peak_acc() { return kPeakAcc; }

}  // namespace ns
