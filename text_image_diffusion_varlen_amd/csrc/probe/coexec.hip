// Measurement aid, not part of the attention library: how VALU work and MFMA
// work from the two waves that share a SIMD slow each other down. Built into
// libmfprobe.so next to the MFMA-rate loop.
//
//   mf_probe_coexec(out, blocks, mode, vkind, mfma_iters, valu_iters, stream)
//     One workgroup of 8 waves per block (2 waves per SIMD on gfx950 when
//     blocks = CU count). Waves 0-3 run mfma_iters iterations of 8 independent
//     v_mfma_f32_16x16x32_bf16 (mode bit 0), waves 4-7 run valu_iters
//     iterations of 16 independent VALU operations (mode bit 1):
//       vkind 0: v_fma_f32            (16 per iteration)
//       vkind 1: v_exp_f32, v_mul_f32 (16 each per iteration)
//       vkind 2: v_maximum3_f32-class max and v_mul_f32 (8 each per iteration)
//     A wave with its bit clear exits at once. Lane 0 of every wave writes its
//     s_memtime stamps (start, end; core clock) to
//     out[2 * (block * 8 + wave) + {0, 1}] (device, 16 * blocks uint64).
//   Returns the hipError_t of the launch.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int VKIND>
__global__ void __launch_bounds__(512, 1)
coexec(unsigned long long* __restrict__ out, int mode, int mfma_iters, int valu_iters, float seed) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  float res = 0.f;
  if (wave < 4) {
    if (mode & 1) {
      bf16x8 a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * float(lane + i));
        b[i] = (__bf16)(seed * float(lane - i));
      }
      f32x4 acc[8];
      for (int i = 0; i < 8; ++i) acc[i] = f32x4{};
#pragma unroll 2
      for (int it = 0; it < mfma_iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
      }
      for (int i = 0; i < 8; ++i) res += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    }
  } else if (mode & 2) {
    float x[16];
    for (int i = 0; i < 16; ++i) x[i] = seed * float(lane + i);
#pragma unroll 4
    for (int it = 0; it < valu_iters; ++it) {
      if constexpr (VKIND == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
      } else if constexpr (VKIND == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * 0.5f;
      } else {
#pragma unroll
        for (int i = 0; i < 16; i += 2)
          x[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[i], x[i + 1]), x[(i + 2) & 15] * 0.999f);
      }
    }
    for (int i = 0; i < 16; ++i) res += x[i];
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    out[2 * (blockIdx.x * 8 + wave)] = t0;
    out[2 * (blockIdx.x * 8 + wave) + 1] = t1;
  }
  if (res == 12345.f) out[0] = 0;  // keeps the work
}

}  // namespace

extern "C" int mf_probe_coexec(unsigned long long* out, int blocks, int mode, int vkind, int mfma_iters,
                               int valu_iters, hipStream_t stream) {
  if (!out || blocks <= 0 || mfma_iters < 0 || valu_iters < 0 || mode < 0 || mode > 3 || vkind < 0 || vkind > 2)
    return int(hipErrorInvalidValue);
  const dim3 grid{unsigned(blocks), 1, 1}, block{512, 1, 1};
  if (vkind == 0) hipLaunchKernelGGL(coexec<0>, grid, block, 0, stream, out, mode, mfma_iters, valu_iters, 0.001f);
  else if (vkind == 1) hipLaunchKernelGGL(coexec<1>, grid, block, 0, stream, out, mode, mfma_iters, valu_iters, 0.001f);
  else hipLaunchKernelGGL(coexec<2>, grid, block, 0, stream, out, mode, mfma_iters, valu_iters, 0.001f);
  return int(hipGetLastError());
}
