// Measurement aid, not part of the attention library: a loop of independent
// bf16 MFMAs on random register operands, no memory traffic, so that the rate
// the chip sustains for each MFMA shape can be reported next to the kernels'
// own rates (same run, same device). Built as libmfprobe.so.
//
//   mf_probe_mfma_loop(out, shape, blocks, iters, stream)
//     shape 0: v_mfma_f32_16x16x32_bf16, 16 independent accumulators per wave
//     shape 1: v_mfma_f32_32x32x16_bf16,  8 independent accumulators per wave
//   Each of the `blocks` workgroups (4 waves) runs `iters` iterations of
//   262144 FLOP per wave (both shapes), then writes one float per thread to
//   out[blocks * 256] (device) so that nothing is optimized away.
//   Returns the hipError_t of the launch.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Eight values uniform in [-1, 1) on the bf16 grid.
__device__ inline bf16x8 operand(uint32_t seed) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float(int(mix(seed * 8u + i) & 0xFFFFu) - 32768) * (1.0f / 32768.0f));
  return r;
}

template <int SHAPE>
__global__ void __launch_bounds__(256, 2) mfma_loop(float* __restrict__ out, int iters) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(t * 8u + i);
    b[i] = operand(t * 8u + 4u + i);
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += acc[i][j][e];
  } else {
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  }
  out[t] = s;
}

}  // namespace

extern "C" int mf_probe_mfma_loop(float* out, int shape, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0 || (shape != 0 && shape != 1)) return int(hipErrorInvalidValue);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_loop<0>, dim3(unsigned(blocks)), dim3(256), 0, stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_loop<1>, dim3(unsigned(blocks)), dim3(256), 0, stream, out, iters);
  return int(hipGetLastError());
}
