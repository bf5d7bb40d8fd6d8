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
// The prologue of the attention path (prologue_bf16_kernel, and
// rope_pack_kernel for fp32) runs one workgroup per (KTILE-row tile of the
// padded layout, head). It rotates the keys (and, for fp32, the queries) of
// every token of the tile and writes into the workspace:
//   Q~  f32 only: [head][row][d] row-major (the bf16 attention kernel rotates
//       its query rows itself while loading them)
//   K~  bf16: each KTILE x d tile stored chunk-major: 16-byte chunk c (channels
//       8c..8c+7) of tile row n at chunk index c * KTILE + n. f32: row-major.
//   V~  bf16: V transposed per tile, [d][KTILE] inside each tile, stored
//       chunk-major: chunk g (8 keys) of channel r at g * d + r, holding keys
//       b..b+3 and b+16..b+19 (b = 32 (g / 4) + 4 (g % 4)), the keys one lane
//       of the 16 x 16 score MFMA's accumulators holds for a 32-key k-step of
//       the P.V product. f32: plain row-major copy.
// Chunk-major tiles are copied verbatim into LDS by the attention kernel;
// there, the 16 lanes that read one MFMA operand row block touch 16
// consecutive chunks (no bank conflicts) and every read is a fixed offset
// from a per-lane base.
// Rows that belong to no token are written as zeros: the padding up to KTILE
// of every sample, and for fp32 also the slack after the last sample (read by
// the last query tile's Q~ rows; the bf16 prologue skips the slack, which no
// bf16 kernel reads).
#include "meta_small.h"
#include "mf_common.h"
#include "rope_math.h"

namespace mf {

// ---------------------------------------------------------------------------
// bf16 prologue. One workgroup per (KTILE-row tile of the padded layout,
// head), the head index fastest. Rows are read whole (16 lanes x 16 B per
// row), keys rotated in fp32, and both tiles staged through LDS: K~ leaves
// chunk-major, V transposed in the score MFMA's key order. Inputs are read
// with element strides (token, head).
//
// FUSED (batches of at most 64 samples): every wave derives the batch's
// offsets itself (one lane per sample, wave scans), and workgroup 0 also
// writes the metadata sections of the workspace for the attention kernel, so
// no separate metadata launch precedes the prologue. Otherwise the metadata
// kernel has run and its sections are read.
struct PrologueArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_st, k_sh, v_st, v_sh;  // element strides between tokens / heads
  const int32_t* grid_hw;
  const int32_t* text_len;
  const int32_t* frames;  // editing samples (R3), else null
  const int32_t* cu_in;   // caller's cu_seqlens (FUSED)
  int32_t n_seg;
  int64_t tokens;
  char* ws;
  int64_t off_len, off_cu, off_pcu, off_tiles;
  uint16_t* kw;
  uint16_t* vw;
  const float2* cs;
  Rope3 r3;
  int32_t heads;
  int64_t rows;
};

// Sample covering padded row r0 of this call: first token u0 of the tile in
// the sample, its length, prompt length, grid and first packed token index.
struct TileSample {
  int32_t u0, L, tl, gh, w;
  int64_t tok0;
};

template <bool R3>
__device__ inline bool fused_tile_sample(const PrologueArgs& a, int64_t r0, TileSample& ts) {
  const int lane = threadIdx.x & 63;
  const int32_t n = a.n_seg;
  const bool mine = lane < n;
  bool ok = true;
  int32_t L = 0, h = 1, w = 1, tl = 0;
  if (mine) {
    L = sample_length(a.grid_hw, a.text_len, R3 ? a.frames : nullptr, lane, ok);
    h = a.grid_hw[2 * lane];
    w = a.grid_hw[2 * lane + 1];
    tl = a.text_len[lane];
  }
  const int64_t incl = wave_inclusive_scan(L);
  const int64_t total = __shfl(incl, 63);
  const int64_t excl = incl - L;
  if (mine && int64_t(a.cu_in[lane]) != excl) ok = false;
  if (lane == 0 && (int64_t(a.cu_in[n]) != total || total != a.tokens || total >= (int64_t(1) << 31))) ok = false;
  if (__any(!ok)) return false;
  const int64_t padded = mine ? round_up(L, KTILE) : 0;
  const int64_t pincl = wave_inclusive_scan(padded);
  const int64_t pexcl = pincl - padded;
  const int64_t ptotal = __shfl(pincl, 63);
  ts = TileSample{0, 0, 0, 1, 1, 0};
  if (r0 < ptotal) {
    const uint64_t before = __ballot(mine && pexcl <= r0);
    const int s = int(__popcll(before)) - 1;  // padded offsets strictly increase
    ts.u0 = int32_t(r0 - __shfl(pexcl, s));
    ts.L = __shfl(L, s);
    ts.tl = __shfl(tl, s);
    ts.gh = __shfl(h, s);
    ts.w = __shfl(w, s);
    ts.tok0 = __shfl(excl, s) + ts.u0;
  }
  return true;
}

template <bool R3>
__device__ inline void ws_tile_sample(const PrologueArgs& a, int64_t r0, TileSample& ts) {
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t* len = reinterpret_cast<const int32_t*>(a.ws + a.off_len);
  const int32_t* cu = reinterpret_cast<const int32_t*>(a.ws + a.off_cu);
  const int32_t* pcu = reinterpret_cast<const int32_t*>(a.ws + a.off_pcu);
  ts = TileSample{0, 0, 0, 1, 1, 0};
  if (r0 < hdr->padded_total) {
    const int32_t s = upper_segment(pcu, hdr->n_seg, r0);
    ts.u0 = int32_t(r0 - pcu[s]);
    ts.L = len[s];
    ts.tok0 = int64_t(cu[s]) + ts.u0;
    ts.tl = a.text_len[s];
    ts.gh = a.grid_hw[2 * s];
    ts.w = a.grid_hw[2 * s + 1];
  }
}

template <int D, bool R3, bool FUSED>
__global__ void __launch_bounds__(256) prologue_bf16_kernel(PrologueArgs a) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CPT = KTILE * CPR;    // chunks per tile
  constexpr int KS = KTILE + 1;       // LDS stride (chunks) between channel chunks: no bank conflicts
  constexpr int VS = D + 2;           // padded LDS row (elements): consecutive keys in different banks
  __shared__ Chunk<uint16_t> ks[CPR * KS];
  __shared__ uint16_t vs[KTILE * VS];
  const int t = threadIdx.x;
  const int h = int(blockIdx.x % unsigned(a.heads));
  const int64_t tile = int64_t(blockIdx.x / unsigned(a.heads));
  const int64_t r0 = tile * KTILE;
  TileSample ts;
  if constexpr (FUSED) {
    if (blockIdx.x == 0 && t < 64) {
      meta_small(a.grid_hw, a.text_len, R3 ? a.frames : nullptr, a.cu_in, a.n_seg, a.tokens,
                 reinterpret_cast<WsHeader*>(a.ws), reinterpret_cast<int32_t*>(a.ws + a.off_len),
                 reinterpret_cast<int32_t*>(a.ws + a.off_cu), reinterpret_cast<int32_t*>(a.ws + a.off_pcu),
                 reinterpret_cast<int2*>(a.ws + a.off_tiles));
    }
    if (!fused_tile_sample<R3>(a, r0, ts)) return;  // same verdict in every wave
  } else {
    if (reinterpret_cast<const WsHeader*>(a.ws)->flag != FLAG_OK) return;
    ws_tile_sample<R3>(a, r0, ts);
  }
  // Tiles past the last sample (the slack rows) are never read by the bf16
  // attention kernel, which visits only its sample's own key tiles.
  if (ts.L == 0) return;
  const int64_t tile_off = (int64_t(h) * a.rows + r0) * D;
  const int64_t tok_base = ts.tok0 - ts.u0;  // packed index of the sample's first token
  // Every thread handles chunks f = t + 256 i of the tile (row f / CPR, channel
  // chunk f % CPR): its K and V chunks and (2D) the four (cos, sin) entries of
  // the K chunk are all loaded before any is used (native vector registers;
  // rows past the sample re-read its last token and are zeroed), then K is
  // rotated and both go to LDS.
  constexpr int PER = CPT / 256;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  u32x4v kr[PER], vr[PER];
  f32x4 tab[R3 ? 1 : PER][2];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = t + 256 * i, rr = f / CPR, cc = f % CPR;
    const int32_t u = min(ts.u0 + rr, ts.L - 1);
    const int64_t row = tok_base + u;
    kr[i] = *reinterpret_cast<const u32x4v*>(a.k + row * a.k_st + int64_t(h) * a.k_sh + cc * 8);
    vr[i] = *reinterpret_cast<const u32x4v*>(a.v + row * a.v_st + int64_t(h) * a.v_sh + cc * 8);
    if constexpr (!R3) {
      int32_t prow, pcol;
      token_position(u, ts.tl, ts.w, prow, pcol);
      const bool first_half = cc < CPR / 2;
      const f32x4* e = reinterpret_cast<const f32x4*>(a.cs + (first_half ? prow : pcol) * (D / 4) +
                                                      4 * (first_half ? cc : cc - CPR / 2));
      tab[i][0] = e[0];
      tab[i][1] = e[1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above in flight before the first use
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = t + 256 * i, rr = f / CPR, cc = f % CPR;
    const int32_t u = ts.u0 + rr;
    Chunk<uint16_t> ko;
    u32x4v vo = vr[i];
    if (u < ts.L) {
      const Chunk<uint16_t> x = __builtin_bit_cast(Chunk<uint16_t>, kr[i]);
      if constexpr (R3) {
        int32_t row, col, frame;
        token_position3(u, ts.tl, ts.gh, ts.w, row, col, frame);
        ko = rotate_chunk3<uint16_t, D>(x, cc * 8, row, col, frame, a.r3);
      } else {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const float c = tab[i][pp >> 1][2 * (pp & 1)], sn = tab[i][pp >> 1][2 * (pp & 1) + 1];
          const float2 y = rotate_pair(bf16_to_f32(x.v[2 * pp]), bf16_to_f32(x.v[2 * pp + 1]), c, sn);
          ko.v[2 * pp] = f32_to_bf16_rne(y.x);
          ko.v[2 * pp + 1] = f32_to_bf16_rne(y.y);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) ko.v[e] = 0;
      vo = u32x4v{0, 0, 0, 0};
    }
    ks[cc * KS + rr] = ko;
    uint32_t* dst = reinterpret_cast<uint32_t*>(vs + rr * VS + cc * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = vo[e];
  }
  __syncthreads();
  // K~ chunk f2 = cc * KTILE + rr (chunk-major).
  for (int f2 = t; f2 < CPT; f2 += 256) {
    const int cc = f2 / KTILE, rr = f2 % KTILE;
    *reinterpret_cast<Chunk<uint16_t>*>(a.kw + tile_off + int64_t(f2) * 8) = ks[cc * KS + rr];
  }
  // V~^T chunk f2 = g * D + c: channel c, keys b..b+3 and b+16..b+19 of the
  // tile (b = 32 (g / 4) + 4 (g % 4): the score MFMA's accumulator order).
  for (int f2 = t; f2 < D * (KTILE / 8); f2 += 256) {
    const int g = f2 / D, c = f2 % D;
    const int b = 32 * (g >> 2) + 4 * (g & 3);
    Chunk<uint16_t> o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o.v[e] = vs[(b + e) * VS + c];
      o.v[4 + e] = vs[(b + 16 + e) * VS + c];
    }
    *reinterpret_cast<Chunk<uint16_t>*>(a.vw + tile_off + int64_t(f2) * 8) = o;
  }
}

// R3: editing samples with frame-aware (row, col, frame) RoPE (r3), else 2D (cs).
template <typename T, int D, bool R3>
__global__ void __launch_bounds__(256)
rope_pack_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
                 const char* __restrict__ ws, int64_t off_len, int64_t off_cu, int64_t off_pcu,
                 T* __restrict__ qw, T* __restrict__ kw, T* __restrict__ vw,
                 const float2* __restrict__ cs, Rope3 r3, int32_t heads, int64_t rows, Strides st) {
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

  // Q~ and K~ rotated, row-major.
  for (int f = threadIdx.x; f < CPT; f += 256) {
    const int rr = f / CPR, cc = f % CPR;
    const int32_t u = u0 + rr;
    Chunk<T> qo, ko;
    if (u < L) {
      qo = rotate(*reinterpret_cast<const Chunk<T>*>(q + (tok0 + rr) * st.q_st + int64_t(h) * st.q_sh + cc * E), cc, u);
      ko = rotate(*reinterpret_cast<const Chunk<T>*>(k + (tok0 + rr) * st.k_st + int64_t(h) * st.k_sh + cc * E), cc, u);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) qo.v[e] = ko.v[e] = T(0);
    }
    *reinterpret_cast<Chunk<T>*>(qw + tile_off + int64_t(f) * E) = qo;
    *reinterpret_cast<Chunk<T>*>(kw + tile_off + int64_t(f) * E) = ko;
  }

  // f32: V copied row-major into the padded layout.
  for (int f = threadIdx.x; f < CPT; f += 256) {
    const int rr = f / CPR, cc = f % CPR;
    Chunk<T> vo;
    if (u0 + rr < L) {
      vo = *reinterpret_cast<const Chunk<T>*>(v + (tok0 + rr) * st.v_st + int64_t(h) * st.v_sh + cc * E);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) vo.v[e] = T(0);
    }
    *reinterpret_cast<Chunk<T>*>(vw + tile_off + int64_t(f) * E) = vo;
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
                                     int32_t heads, const Strides& st, hipStream_t s) {
  char* w = const_cast<char*>(ws);
  dim3 grid(unsigned(l.rows / KTILE), unsigned(heads));
  hipLaunchKernelGGL((rope_pack_kernel<T, D, R3>), grid, dim3(256), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     grid_hw, text_len, ws, l.off_len, l.off_cu, l.off_pcu,
                     reinterpret_cast<T*>(w + l.off_q), reinterpret_cast<T*>(w + l.off_k),
                     reinterpret_cast<T*>(w + l.off_v), cs, r3, heads, l.rows, st);
  return hipGetLastError();
}

template <typename T, bool R3>
static hipError_t launch_rope_pack_d(const void* q, const void* k, const void* v, const int32_t* grid_hw,
                                     const int32_t* text_len, const char* ws, const WsLayout& l,
                                     const float2* cs, Rope3 r3, int32_t heads, int32_t head_dim,
                                     const Strides& st, hipStream_t s) {
  return head_dim == 128 ? launch_rope_pack_t<T, 128, R3>(q, k, v, grid_hw, text_len, ws, l, cs, r3, heads, st, s)
                         : launch_rope_pack_t<T, 64, R3>(q, k, v, grid_hw, text_len, ws, l, cs, r3, heads, st, s);
}

// bf16 prologue: fused with the metadata derivation (n_seg <= 64) or after
// meta_kernel. k, v with element strides (token, head).
hipError_t launch_prologue_bf16(const void* k, int64_t k_st, int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh,
                                const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                const int32_t* cu_in, int32_t n_seg, int64_t tokens, char* ws, const WsLayout& l,
                                const float2* cs, const Rope3* r3, int32_t heads, int32_t head_dim, bool fused,
                                hipStream_t s) {
  PrologueArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_st = k_st;
  a.k_sh = k_sh;
  a.v_st = v_st;
  a.v_sh = v_sh;
  a.grid_hw = grid_hw;
  a.text_len = text_len;
  a.frames = frames;
  a.cu_in = cu_in;
  a.n_seg = n_seg;
  a.tokens = tokens;
  a.ws = ws;
  a.off_len = l.off_len;
  a.off_cu = l.off_cu;
  a.off_pcu = l.off_pcu;
  a.off_tiles = l.off_tiles;
  a.kw = reinterpret_cast<uint16_t*>(ws + l.off_k);
  a.vw = reinterpret_cast<uint16_t*>(ws + l.off_v);
  a.cs = cs;
  a.r3 = r3 ? *r3 : Rope3{nullptr, 0, 0};
  a.heads = heads;
  a.rows = l.rows;
  const dim3 grid(unsigned(l.rows / KTILE * heads));
#define MF_PROLOGUE(D, R3, F) hipLaunchKernelGGL((prologue_bf16_kernel<D, R3, F>), grid, dim3(256), 0, s, a)
  if (head_dim == 128) {
    if (r3) { if (fused) MF_PROLOGUE(128, true, true); else MF_PROLOGUE(128, true, false); }
    else { if (fused) MF_PROLOGUE(128, false, true); else MF_PROLOGUE(128, false, false); }
  } else {
    if (r3) { if (fused) MF_PROLOGUE(64, true, true); else MF_PROLOGUE(64, true, false); }
    else { if (fused) MF_PROLOGUE(64, false, true); else MF_PROLOGUE(64, false, false); }
  }
#undef MF_PROLOGUE
  return hipGetLastError();
}

// f32 prologue (after meta_kernel). r3 == nullptr: 2D RoPE with the table cs;
// else frame-aware RoPE.
hipError_t launch_rope_pack(const void* q, const void* k, const void* v, const int32_t* grid_hw,
                            const int32_t* text_len, const char* ws, const WsLayout& l,
                            const float2* cs, const Rope3* r3, int32_t heads, int32_t head_dim, const Strides& st,
                            hipStream_t s) {
  const Rope3 r = r3 ? *r3 : Rope3{nullptr, 0, 0};
  return r3 ? launch_rope_pack_d<float, true>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, st, s)
            : launch_rope_pack_d<float, false>(q, k, v, grid_hw, text_len, ws, l, cs, r, heads, head_dim, st, s);
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
