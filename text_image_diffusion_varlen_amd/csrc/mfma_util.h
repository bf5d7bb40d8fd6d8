// Register-level helpers shared by the MFMA attention kernels (forward and
// backward): bf16 operand types, packing, cross-half row reductions and the
// direct-to-LDS tile copy.
#pragma once

#include "mf_common.h"

namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// D (32 x 32, fp32) += A (32 x 16, bf16) B (16 x 32, bf16). Lane l supplies
// A row l % 32 and B column l % 32, k = 8 (l / 32) .. +7 of each; it receives
// D column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4 in entry e.
__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D (16 x 16, fp32) += A (16 x 32, bf16) B (32 x 16, bf16). Lane l supplies A
// row l % 16 and B column l % 16, k = 8 (l / 16) .. +7 of each; it receives D
// column l % 16, rows 4 (l / 16) .. +3. On gfx950 this form sustains a higher
// rate than the 32 x 32 x 16 one (about 14 % more in a loop of independent
// MFMAs on random register operands).
__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// Combine a value with the same register of lane ^ 32. v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second; with both operands equal to x, every lane ends up holding x[l]
// in one result and x[l ^ 32] in the other, so a symmetric combine of the two
// results needs no lane test.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// acc + p0 + p1 for a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).
__device__ inline float dot2_bf16_sum(uint32_t pair, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// Raw buffer resource over `bytes` bytes at p (no stride, no format
// conversion; lanes past the range read zeros).
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Copies CHUNKS consecutive 16-byte chunks from global memory into LDS with
// gfx950 direct-to-LDS loads: each of WAVES waves moves CHUNKS / WAVES chunks,
// one contiguous 1 KB per instruction, without passing through registers.
// The loads are buffer loads (MUBUF), not global (FLAT) ones: the compiler
// treats a FLAT load into LDS as pending on both memory counters, and while
// one is in flight every LDS-read wait it places becomes a full drain
// (lgkmcnt(0)); with the buffer form it keeps exact counts, so operand reads
// stay pipelined behind the copies. src must be the same in every lane.
template <int CHUNKS, int WAVES>
__device__ inline void copy_to_lds(const u32x4* __restrict__ src, u32x4* dst, int wave, int lane) {
  constexpr int PER_WAVE = CHUNKS / WAVES;
  static_assert(PER_WAVE % 64 == 0, "whole 1 KB copies per wave");
  const __amdgpu_buffer_rsrc_t rs = raw_rsrc(src, CHUNKS * 16);
#pragma unroll
  for (int i = 0; i < PER_WAVE / 64; ++i) {
    const int c = wave * PER_WAVE + i * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + c), 16, (c + lane) * 16, 0, 0, 0);
  }
}

// This wave's outstanding vector-memory operations (including direct-to-LDS
// copies) have completed, then a workgroup barrier.
__device__ inline void wait_vm_and_sync() {
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __syncthreads();
}

}  // namespace mf
