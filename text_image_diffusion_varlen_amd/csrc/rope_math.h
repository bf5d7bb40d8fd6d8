// 2D RoPE arithmetic shared by the prologue, the standalone RoPE kernel and
// the attention kernel (which rotates its query rows as it loads them).
// Layout: channels [0, d/2) turn by the row, [d/2, d) by the column; adjacent
// pairs (2j, 2j+1) inside each half at frequency theta^(-2j/(d/2)), read from a
// float2 cos/sin table [ROPE_PMAX][d/4]; (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).
#pragma once

#include "mf_common.h"

namespace mf {

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int PER_CHUNK = 8;
  __device__ static float load(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t store(float x) { return f32_to_bf16_rne(x); }
};
template <> struct Elem<float> {
  static constexpr int PER_CHUNK = 4;
  __device__ static float load(float x) { return x; }
  __device__ static float store(float x) { return x; }
};

template <typename T> struct alignas(16) Chunk { T v[16 / sizeof(T)]; };

// One channel pair turned by the angle with cosine c and sine s:
// (x0, x1) -> (x0 c - x1 s, x0 s + x1 c). The fused multiply-adds are written
// out so that every kernel that rotates (prologue, query load, standalone
// RoPE, 2D and frame-aware tables) rounds identically.
__device__ inline float2 rotate_pair(float x0, float x1, float c, float s) {
  return make_float2(__builtin_fmaf(x0, c, -(x1 * s)), __builtin_fmaf(x0, s, x1 * c));
}

// Rotates one 16-byte chunk (channels d0 .. d0+E-1, E even) of a row at (row, col);
// with SCALED, each rotated value is also multiplied by `scale` before it is stored.
template <typename T, int D, bool SCALED = false>
__device__ inline Chunk<T> rotate_chunk(const Chunk<T>& in, int d0, int32_t row, int32_t col,
                                        const float2* __restrict__ cs, float scale = 1.f) {
  constexpr int E = Elem<T>::PER_CHUNK;
  Chunk<T> out;
#pragma unroll
  for (int pp = 0; pp < E / 2; ++pp) {
    const int d = d0 + 2 * pp;
    const bool first_half = d < D / 2;
    const int j = first_half ? d / 2 : (d - D / 2) / 2;
    const int32_t p = first_half ? row : col;
    const float2 r = cs[p * (D / 4) + j];
    const float x0 = Elem<T>::load(in.v[2 * pp]);
    const float x1 = Elem<T>::load(in.v[2 * pp + 1]);
    const float2 y = rotate_pair(x0, x1, r.x, r.y);
    out.v[2 * pp] = Elem<T>::store(SCALED ? y.x * scale : y.x);
    out.v[2 * pp + 1] = Elem<T>::store(SCALED ? y.y * scale : y.y);
  }
  return out;
}

// Frame-aware RoPE (editing samples: (row, col, frame) positions). Channel
// pairs k = 0 .. D/2-1 in three contiguous blocks: [0, b1) turn by the row,
// [b1, b2) by the column, [b2, D/2) by the frame; each block has its own
// frequency ladder theta^(-2j/m), m = channels of the block. The cos/sin
// table is [ROPE_PMAX][D/2], entry (p, k) = cos/sin of p times pair k's
// frequency, computed on the host in double precision.
struct Rope3 {
  const float2* cs;
  int32_t b1, b2;
};

__device__ inline float2 rope3_cs(const Rope3& r, int D, int k, int32_t row, int32_t col, int32_t frame) {
  const int32_t p = k < r.b1 ? row : (k < r.b2 ? col : frame);
  return r.cs[p * (D / 2) + k];
}

template <typename T, int D, bool SCALED = false>
__device__ inline Chunk<T> rotate_chunk3(const Chunk<T>& in, int d0, int32_t row, int32_t col, int32_t frame,
                                         const Rope3& r, float scale = 1.f) {
  constexpr int E = Elem<T>::PER_CHUNK;
  Chunk<T> out;
#pragma unroll
  for (int pp = 0; pp < E / 2; ++pp) {
    const float2 c = rope3_cs(r, D, d0 / 2 + pp, row, col, frame);
    const float x0 = Elem<T>::load(in.v[2 * pp]);
    const float x1 = Elem<T>::load(in.v[2 * pp + 1]);
    const float2 y = rotate_pair(x0, x1, c.x, c.y);
    out.v[2 * pp] = Elem<T>::store(SCALED ? y.x * scale : y.x);
    out.v[2 * pp + 1] = Elem<T>::store(SCALED ? y.y * scale : y.y);
  }
  return out;
}

}  // namespace mf
