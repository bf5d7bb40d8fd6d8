// 2D rotary position embedding on the device.
//
// Source: mageflow.net architecture page, section 2 (2D RoPE encodes the 2D
// spatial position of every latent token natively, any aspect ratio, with no
// interpolation onto a fixed grid). Layout taken: channels [0, d/2) turn by
// the row, [d/2, d) by the column; adjacent pairs (2j, 2j+1) inside each half
// at frequency theta^(-2j/(d/2)); (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).
// Prompt tokens sit at (0, 0) and are therefore left unrotated.
//
// cos/sin come from a float2 table [ROPE_PMAX][d/4] computed on the host in
// double precision (entry (p, j) = cos/sin of p * theta^(-2j/(d/2))); the
// device does the rotation in fp32.
//
// Editing samples (tech report, NR-MMDiT editing paragraph) use the
// frame-aware variant: (row, col, frame) positions, three channel blocks
// (rope_math.h, Rope3).
//
// rope_pack_kernel is the prologue of the attention path. One workgroup per
// (KTILE-row tile of the padded layout, head). It rotates the keys (and, for
// f32, the queries) of every token of the tile and writes into the workspace:
//   Q~  f32 only: [head][row][d] row-major (the bf16 attention kernel rotates
//       its query rows itself while loading them)
//   K~  bf16: each KTILE x d tile stored chunk-major: 16-byte chunk c (channels
//       8c..8c+7) of tile row n at chunk index c * KTILE + n. f32: row-major.
//   V~  bf16: V transposed per tile, [d][KTILE] inside each tile, keys inside
//       every group of 16 stored in the order 0-3, 8-11, 4-7, 12-15 (the order
//       in which the MFMA accumulator of the score tile holds them), and the
//       tile stored chunk-major: chunk g (8 keys) of channel r at g * d + r.
//       f32: plain row-major copy.
// Chunk-major tiles are copied verbatim into LDS by the attention kernel;
// there, the 16 lanes that read one MFMA operand row block touch 16
// consecutive chunks (no bank conflicts) and every read is a fixed offset
// from a per-lane base.
// Rows that belong to no token (padding up to KTILE, and the slack after the
// last sample) are written as zeros.
#include "mf_common.h"
#include "rope_math.h"

namespace mf {

// R3: editing samples with frame-aware (row, col, frame) RoPE (r3), else 2D (cs).
template <typename T, int D, bool R3>
__global__ void __launch_bounds__(256)
rope_pack_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
                 const char* __restrict__ ws, int64_t off_len, int64_t off_cu, int64_t off_pcu,
                 T* __restrict__ qw, T* __restrict__ kw, T* __restrict__ vw,
                 const float2* __restrict__ cs, Rope3 r3, int32_t heads, int64_t rows) {
  constexpr int E = Elem<T>::PER_CHUNK;
  constexpr int CPR = D / E;             // chunks per row
  constexpr int CPT = KTILE * CPR;       // chunks per tile
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t* len = reinterpret_cast<const int32_t*>(ws + off_len);
  const int32_t* cu = reinterpret_cast<const int32_t*>(ws + off_cu);
  const int32_t* pcu = reinterpret_cast<const int32_t*>(ws + off_pcu);

  const int64_t r0 = int64_t(blockIdx.x) * KTILE;
  const int h = blockIdx.y;
  const int32_t n = hdr->n_seg;
  int32_t u0 = 0, L = 0, tl = 0, w = 1, gh = 1;
  int64_t tok0 = 0;
  if (r0 < hdr->padded_total) {
    const int32_t s = upper_segment(pcu, n, r0);
    u0 = int32_t(r0 - pcu[s]);
    L = len[s];
    tok0 = int64_t(cu[s]) + u0;
    tl = text_len[s];
    gh = grid_hw[2 * s];
    w = grid_hw[2 * s + 1];
  }
  // Rotation of chunk cc (channels cc*E ..) of sample token u.
  auto rotate = [&](const Chunk<T>& x, int cc, int32_t u) {
    if constexpr (R3) {
      int32_t row, col, frame;
      token_position3(u, tl, gh, w, row, col, frame);
      return rotate_chunk3<T, D>(x, cc * E, row, col, frame, r3);
    } else {
      int32_t row, col;
      token_position(u, tl, w, row, col);
      return rotate_chunk<T, D>(x, cc * E, row, col, cs);
    }
  };
  const int64_t tile_off = (int64_t(h) * rows + r0) * D;
  const int64_t src_stride = int64_t(heads) * D;  // elements between consecutive tokens

  if constexpr (sizeof(T) == 4) {
    // f32: Q~ and K~ rotated, row-major.
    for (int f = threadIdx.x; f < CPT; f += 256) {
      const int rr = f / CPR, cc = f % CPR;
      const int32_t u = u0 + rr;
      Chunk<T> qo, ko;
      if (u < L) {
        const int64_t src = (tok0 + rr) * src_stride + int64_t(h) * D + cc * E;
        qo = rotate(*reinterpret_cast<const Chunk<T>*>(q + src), cc, u);
        ko = rotate(*reinterpret_cast<const Chunk<T>*>(k + src), cc, u);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) qo.v[e] = ko.v[e] = T(0);
      }
      *reinterpret_cast<Chunk<T>*>(qw + tile_off + int64_t(f) * E) = qo;
      *reinterpret_cast<Chunk<T>*>(kw + tile_off + int64_t(f) * E) = ko;
    }
  }

  if constexpr (sizeof(T) == 4) {
    // f32: V copied row-major into the padded layout.
    for (int f = threadIdx.x; f < CPT; f += 256) {
      const int rr = f / CPR, cc = f % CPR;
      Chunk<T> vo;
      if (u0 + rr < L) {
        vo = *reinterpret_cast<const Chunk<T>*>(v + (tok0 + rr) * src_stride + int64_t(h) * D + cc * E);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) vo.v[e] = T(0);
      }
      *reinterpret_cast<Chunk<T>*>(vw + tile_off + int64_t(f) * E) = vo;
    }
  } else {
    // bf16 (queries are rotated by the attention kernel itself): the K tile is
    // rotated and staged through LDS, then written chunk-major; the V tile goes
    // through LDS and is written transposed ([d][KTILE]) in MFMA key order.
    // Loads read whole rows (16 lanes x 16 B), stores write consecutive chunks.
    constexpr int KS = KTILE + 1;  // LDS stride (chunks) between channel chunks: no bank conflicts
    constexpr int VS = D + 2;      // padded LDS row (elements): consecutive keys fall in different banks
    __shared__ Chunk<T> ks[CPR * KS];
    __shared__ uint16_t vs[KTILE * VS];
    for (int f = threadIdx.x; f < CPT; f += 256) {
      const int rr = f / CPR, cc = f % CPR;
      const int32_t u = u0 + rr;
      Chunk<T> ko, vi;
      if (u < L) {
        const int64_t src = (tok0 + rr) * src_stride + int64_t(h) * D + cc * E;
        ko = rotate(*reinterpret_cast<const Chunk<T>*>(k + src), cc, u);
        vi = *reinterpret_cast<const Chunk<T>*>(v + src);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) ko.v[e] = vi.v[e] = T(0);
      }
      ks[cc * KS + rr] = ko;
      uint32_t* dst = reinterpret_cast<uint32_t*>(vs + rr * VS + cc * E);
      const uint32_t* sv = reinterpret_cast<const uint32_t*>(vi.v);
#pragma unroll
      for (int e = 0; e < E / 2; ++e) dst[e] = sv[e];
    }
    __syncthreads();
    // K~ chunk f2 = cc * KTILE + rr (chunk-major).
    for (int f2 = threadIdx.x; f2 < CPT; f2 += 256) {
      const int cc = f2 / KTILE, rr = f2 % KTILE;
      *reinterpret_cast<Chunk<T>*>(kw + tile_off + int64_t(f2) * E) = ks[cc * KS + rr];
    }
    __syncthreads();
    // Output chunk f2 = g * D + c: channel c, keys of chunk g of the 64-key row.
    for (int f2 = threadIdx.x; f2 < D * (KTILE / 8); f2 += 256) {
      const int g = f2 / D, c = f2 % D;
      const int base = 16 * (g >> 1) + 4 * (g & 1);
      Chunk<T> o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o.v[e] = vs[(base + e) * VS + c];
        o.v[4 + e] = vs[(base + 8 + e) * VS + c];
      }
      *reinterpret_cast<Chunk<T>*>(vw + tile_off + int64_t(f2) * 8) = o;
    }
  }
}

// Standalone RoPE: x_out = R(pos) x_in for [tokens][heads][D]; pos is
// [tokens][2] (2D) or [tokens][3] (R3: row, col, frame). Positions outside
// [0, ROPE_PMAX) copy the row unchanged and flag FLAG_POSITION.
template <typename T, int D, bool R3>
__global__ void __launch_bounds__(256)
rope_kernel(const T* __restrict__ x, T* __restrict__ y, const int32_t* __restrict__ pos,
            int64_t tokens, int32_t heads, const float2* __restrict__ cs, Rope3 r3, int32_t* status) {
  constexpr int E = Elem<T>::PER_CHUNK;
  constexpr int CPR = D / E;
  constexpr int NP = R3 ? 3 : 2;
  const int64_t f = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (f >= tokens * heads * CPR) return;
  const int64_t t = f / (int64_t(heads) * CPR);
  const int cc = int(f % CPR);
  const int32_t row = pos[NP * t], col = pos[NP * t + 1], frame = R3 ? pos[NP * t + 2] : 0;
  const Chunk<T> in = *reinterpret_cast<const Chunk<T>*>(x + f * E);
  Chunk<T> out;
  if (row < 0 || col < 0 || frame < 0 || row >= ROPE_PMAX || col >= ROPE_PMAX || frame >= ROPE_PMAX) {
    out = in;
    if (cc == 0) atomicOr(status, FLAG_POSITION);
  } else if constexpr (R3) {
    out = rotate_chunk3<T, D>(in, cc * E, row, col, frame, r3);
  } else {
    out = rotate_chunk<T, D>(in, cc * E, row, col, cs);
  }
  *reinterpret_cast<Chunk<T>*>(y + f * E) = out;
}

template <typename T, int D, bool R3>
static hipError_t launch_rope_pack_t(const void* q, const void* k, const void* v,
                                     const int32_t* grid_hw, const int32_t* text_len,
                                     const char* ws, const WsLayout& l, const float2* cs, Rope3 r3,
                                     int32_t heads, hipStream_t s) {
  char* w = const_cast<char*>(ws);
  dim3 grid(unsigned(l.rows / KTILE), unsigned(heads));
  hipLaunchKernelGGL((rope_pack_kernel<T, D, R3>), grid, dim3(256), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     grid_hw, text_len, ws, l.off_len, l.off_cu, l.off_pcu,
                     reinterpret_cast<T*>(w + l.off_q), reinterpret_cast<T*>(w + l.off_k),
                     reinterpret_cast<T*>(w + l.off_v), cs, r3, heads, l.rows);
  return hipGetLastError();
}

template <typename T, bool R3>
static hipError_t launch_rope_pack_d(const void* q, const void* k, const void* v, const int32_t* grid_hw,
                                     const int32_t* text_len, const char* ws, const WsLayout& l,
                                     const float2* cs, Rope3 r3, int32_t heads, int32_t head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_rope_pack_t<T, 128, R3>(q, k, v, grid_hw, text_len, ws, l, cs, r3, heads, s)
                         : launch_rope_pack_t<T, 64, R3>(q, k, v, grid_hw, text_len, ws, l, cs, r3, heads, s);
}

// r3 == nullptr: 2D RoPE with the table cs; else frame-aware RoPE.
hipError_t launch_rope_pack(const void* q, const void* k, const void* v, const int32_t* grid_hw,
                            const int32_t* text_len, const char* ws, const WsLayout& l,
                            const float2* cs, const Rope3* r3, int32_t heads, int32_t head_dim, bool bf16,
                            hipStream_t s) {
  const Rope3 r = r3 ? *r3 : Rope3{nullptr, 0, 0};
  if (bf16) {
    return r3 ? launch_rope_pack_d<uint16_t, true>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, s)
              : launch_rope_pack_d<uint16_t, false>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, s);
  }
  return r3 ? launch_rope_pack_d<float, true>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, s)
            : launch_rope_pack_d<float, false>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, s);
}

template <typename T, int D, bool R3>
static hipError_t launch_rope_t(const void* x, void* y, const int32_t* pos, int64_t tokens,
                                int32_t heads, const float2* cs, Rope3 r3, int32_t* status, hipStream_t s) {
  constexpr int CPR = D / Elem<T>::PER_CHUNK;
  const int64_t chunks = tokens * heads * CPR;
  hipLaunchKernelGGL((rope_kernel<T, D, R3>), dim3(unsigned(ceil_div(chunks, 256))), dim3(256), 0, s,
                     static_cast<const T*>(x), static_cast<T*>(y), pos, tokens, heads, cs, r3, status);
  return hipGetLastError();
}

template <bool R3>
static hipError_t launch_rope_r(const void* x, void* y, const int32_t* pos, int64_t tokens, int32_t heads,
                                int32_t head_dim, bool bf16, const float2* cs, Rope3 r3, int32_t* status,
                                hipStream_t s) {
  if (bf16) {
    return head_dim == 128 ? launch_rope_t<uint16_t, 128, R3>(x, y, pos, tokens, heads, cs, r3, status, s)
                           : launch_rope_t<uint16_t, 64, R3>(x, y, pos, tokens, heads, cs, r3, status, s);
  }
  return head_dim == 128 ? launch_rope_t<float, 128, R3>(x, y, pos, tokens, heads, cs, r3, status, s)
                         : launch_rope_t<float, 64, R3>(x, y, pos, tokens, heads, cs, r3, status, s);
}

// r3 == nullptr: 2D positions [tokens][2] with table cs; else [tokens][3].
hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t tokens, int32_t heads,
                       int32_t head_dim, bool bf16, const float2* cs, const Rope3* r3, int32_t* status,
                       hipStream_t s) {
  if (r3) return launch_rope_r<true>(x, y, pos, tokens, heads, head_dim, bf16, cs, *r3, status, s);
  return launch_rope_r<false>(x, y, pos, tokens, heads, head_dim, bf16, cs, Rope3{nullptr, 0, 0}, status, s);
}

}  // namespace mf
