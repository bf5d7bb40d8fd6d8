// Packed joint attention backward on gfx950.
//
// Gradients of O = softmax(X) V, X = scale * Q~ K~^T, per sample and head
// (the packed samples are independent: Mage-Flow tech report, NR-MMDiT
// section, per-sample cumulative offsets; training runs on such packed
// batches, same section). With P = softmax(X), the upstream gradient dO and
// D_q = sum_c dO[q][c] O[q][c]:
//   dV = P^T dO,  dP = dO V^T,  dX = P * (dP - D),
//   dQ~ = scale * dX K~,  dK~ = scale * dX^T Q~,
// and the 2D RoPE rotation (orthogonal, mageflow.net architecture page,
// section 2) is undone on dQ~, dK~: dq = R(pos)^T dQ~, dk = R(pos)^T dK~.
// P is recomputed from the forward's saved row log-sum-exp (natural log,
// [heads][tokens]); no score matrix is stored.
//
// Kernels:
//   bwd_pack_kernel  one workgroup per (KTILE padded rows, head): rotates q and
//                    k, and writes Q~, dO, K~, V chunk-major, Q~^T, dO^T, K~^T
//                    in MFMA order (as the forward's V~^T) and per-row
//                    log2-domain LSE and D into the backward workspace.
//   bwd_kv_kernel    one workgroup per (128 keys of a sample, head), 8 waves:
//                    each 32-key group has a dV wave (S, P, dV^T += dO^T P)
//                    and a dK wave (dP, dX, dK^T += Q~^T dX) that receives P
//                    through LDS, so two waves per SIMD fit in registers and
//                    nothing is computed twice; keys resident in registers;
//                    loops over all the sample's 64-query tiles
//                    (double-buffered in LDS); lane = key, entries = queries.
//   bwd_q_kernel     one workgroup per (256 queries of a sample, head), 8 waves
//                    x 32 queries, queries resident in registers; loops over
//                    the sample's 64-key tiles:
//                      S^T = K~ Q~^T, dP^T = V dO^T (lane = query),
//                      dQ^T += K~^T dX^T.
// When the last round of either kernel's units would fill the device poorly
// and the units are long, those units run as pieces (dK/dV over query ranges,
// dQ over key ranges) that write fp32 partial sums to slots of the workspace;
// extra workgroups of bwd_q_kernel merge the dK/dV pieces and
// bwd_q_merge_kernel the dQ pieces, adding them in piece order before the
// usual epilogue (the plans are derived identically on the device from the
// tile table, nothing is stored).
// Every product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P
// and dX are rounded to bf16 (RNE) as MFMA operands. No atomics and a fixed
// summation order everywhere, so results are deterministic.
#include "mf_common.h"
#include "mfma_util.h"
#include "rope_math.h"

namespace mf {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int KV_WAVES = 8;                 // waves of bwd_kv_kernel
constexpr int KV_GROUPS = KV_WAVES / 2;     // 32-key groups: one dV wave and one dK wave each
constexpr int KV_KEYS = 32 * KV_GROUPS;     // keys per bwd_kv workgroup
static_assert(KV_KEYS == BWD_KV_KEYS, "partial slots of the workspace hold KV_KEYS keys");
constexpr int KV_SPLIT = QTILE / KV_KEYS;   // key blocks per entry of the tile table
constexpr int Q_WAVES = QTILE / 32;         // waves of bwd_q_kernel, 32 queries each
static_assert(QTILE % KV_KEYS == 0, "whole key blocks per entry of the tile table");

struct BwdArgs {
  const char* ws;
  int64_t off_len, off_cu, off_pcu, off_tiles;
  const uint16_t* q;     // caller tensors [tokens][heads][d]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;      // [heads][tokens], natural log
  const int32_t* grid_hw;
  const int32_t* text_len;
  const float2* cs;      // cos/sin table [ROPE_PMAX][d/4]
  Rope3 r3;              // frame-aware RoPE of editing samples (R3 kernels)
  uint16_t* qc;
  uint16_t* qt;
  uint16_t* oc;
  uint16_t* ot;
  uint16_t* kc;
  uint16_t* kt;
  uint16_t* vc;
  float* st;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* part;       // partial dV, dK of split dK/dV units, PART_SLOTS slots
  float* qpart;      // partial dQ of split dQ units, PART_SLOTS slots
  int32_t ncu;       // compute units for the dK/dV split plan (0: never split)
  int32_t ncu_q;     // compute units for the dQ split plan (0: never split)
  int64_t dq_units;  // workgroups of the dQ kernel's own grid (units and pieces); dK/dV merges follow
  int32_t heads;
  int64_t rows;      // padded rows per head
  int64_t tokens;
  float c_log2;      // scale * log2(e)
  float scale;
};

// ---------------------------------------------------------------- prologue

template <int D, bool R3>
__global__ void __launch_bounds__(256) bwd_pack_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int CPT = KTILE * CPR;       // chunks per tile
  constexpr int VS = D + 2;              // staged row stride (elements): column reads hit distinct banks
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t* len = reinterpret_cast<const int32_t*>(a.ws + a.off_len);
  const int32_t* cu = reinterpret_cast<const int32_t*>(a.ws + a.off_cu);
  const int32_t* pcu = reinterpret_cast<const int32_t*>(a.ws + a.off_pcu);

  const int64_t r0 = int64_t(blockIdx.x) * KTILE;
  const int h = blockIdx.y;
  int32_t u0 = 0, L = 0, tl = 0, w = 1, gh = 1;
  int64_t tok0 = 0;
  if (r0 < hdr->padded_total) {
    const int32_t s = upper_segment(pcu, hdr->n_seg, r0);
    u0 = int32_t(r0 - pcu[s]);
    L = len[s];
    tok0 = int64_t(cu[s]) + u0;
    tl = a.text_len[s];
    gh = a.grid_hw[2 * s];
    w = a.grid_hw[2 * s + 1];
  }
  const int64_t tile_off = (int64_t(h) * a.rows + r0) * D;  // element offset of this tile
  const int64_t stride = int64_t(a.heads) * D;              // elements between tokens
  __shared__ uint16_t tile[KTILE * VS];
  __shared__ float dsum[KTILE];
  const int tid = threadIdx.x;

  // Stage a KTILE x D tile of `src` (rotated when asked) into LDS; zero rows
  // past the sample. For dO also form D = rowsum(dO * O) (the CPR threads of
  // one row are consecutive lanes, 64 % CPR == 0).
  auto stage = [&](const uint16_t* src, bool rotate, bool with_dsum) {
#pragma unroll
    for (int i = 0; i < CPT / 256; ++i) {
      const int f = tid + 256 * i;
      const int rr = f / CPR, cc = f % CPR;
      const int32_t u = u0 + rr;
      Chunk<uint16_t> x;
      float part = 0.f;
      if (u < L) {
        const int64_t off = (tok0 + rr) * stride + int64_t(h) * D + cc * 8;
        x = *reinterpret_cast<const Chunk<uint16_t>*>(src + off);
        if (rotate) {
          if constexpr (R3) {
            int32_t row, col, frame;
            token_position3(u, tl, gh, w, row, col, frame);
            x = rotate_chunk3<uint16_t, D>(x, cc * 8, row, col, frame, a.r3);
          } else {
            int32_t row, col;
            token_position(u, tl, w, row, col);
            x = rotate_chunk<uint16_t, D>(x, cc * 8, row, col, a.cs);
          }
        }
        if (with_dsum) {
          const Chunk<uint16_t> y = *reinterpret_cast<const Chunk<uint16_t>*>(a.o + off);
#pragma unroll
          for (int e = 0; e < 8; ++e) part = __builtin_fmaf(bf16_to_f32(x.v[e]), bf16_to_f32(y.v[e]), part);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x.v[e] = 0;
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(tile + rr * VS + cc * 8);
      const uint32_t* sv = reinterpret_cast<const uint32_t*>(x.v);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = sv[e];
      if (with_dsum) {
#pragma unroll
        for (int o = CPR / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
        if (cc == 0) dsum[rr] = part;
      }
    }
    __syncthreads();
  };
  // Chunk f2 = c * KTILE + n holds channels 8c .. 8c+7 of row n.
  auto write_chunk_major = [&](uint16_t* dst) {
    for (int f2 = tid; f2 < CPT; f2 += 256) {
      const int cc = f2 / KTILE, rr = f2 % KTILE;
      const uint32_t* sv = reinterpret_cast<const uint32_t*>(tile + rr * VS + cc * 8);
      u32x4 o = {sv[0], sv[1], sv[2], sv[3]};
      *reinterpret_cast<u32x4*>(dst + tile_off + int64_t(f2) * 8) = o;
    }
  };
  // Transposed tile [D][KTILE], rows inside every group of 16 in the order
  // 0-3, 8-11, 4-7, 12-15, chunk-major: chunk g (8 rows) of channel c at g * D + c.
  auto write_transposed = [&](uint16_t* dst) {
    for (int f2 = tid; f2 < D * (KTILE / 8); f2 += 256) {
      const int g = f2 / D, c = f2 % D;
      const int base = 16 * (g >> 1) + 4 * (g & 1);
      Chunk<uint16_t> o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o.v[e] = tile[(base + e) * VS + c];
        o.v[4 + e] = tile[(base + 8 + e) * VS + c];
      }
      *reinterpret_cast<Chunk<uint16_t>*>(dst + tile_off + int64_t(f2) * 8) = o;
    }
  };

  stage(a.q, true, false);
  write_chunk_major(a.qc);
  write_transposed(a.qt);
  __syncthreads();
  stage(a.k, true, false);
  write_chunk_major(a.kc);
  write_transposed(a.kt);
  __syncthreads();
  stage(a.dout, false, true);
  write_chunk_major(a.oc);
  write_transposed(a.ot);
  __syncthreads();
  stage(a.v, false, false);
  write_chunk_major(a.vc);
  if (tid < KTILE) {
    const int32_t u = u0 + tid;
    float* st = a.st + (int64_t(h) * a.rows + r0) * 2;  // tile index * 2 * KTILE
    st[tid] = u < L ? a.lse[int64_t(h) * a.tokens + tok0 + tid] * LOG2E : INFINITY;
    st[KTILE + tid] = u < L ? dsum[tid] : 0.f;
  }
}

// ---------------------------------------------------------------- dK, dV

template <int D>
struct BwdTile {
  static constexpr int CH = KTILE * D / 8;  // 16-byte chunks per KTILE x D tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

// One 64-query tile for one 32-key group, split over the group's two waves
// and two phases with a workgroup barrier between them. T: LDS tile set
// [qc | oc | qt | ot | stats]; pl: this group's P exchange slot (4 KB).
// Entry e of a 32-query half qb of a product with lane = key l32 is query
// 32qb + 8(e/4) + 4hf + e%4; k-step kk of half qb (queries 32qb + 16kk .. +15)
// of the B operands takes entries 8kk .. 8kk+7, which are the queries the
// MFMA-order tiles (qt, ot) hold in chunk 2(2qb + kk) + hf.
//   dV wave, phase 1: S = Q~ K~^T, P = 2^(S c - lse2) packed to bf16, kept in
//                     registers and stored to pl.
//   dK wave, phase 1: dP = dO V^T (kept in registers).
//   dV wave, phase 2: dV^T += dO^T P.
//   dK wave, phase 2: P from pl, dX = P (dP - D) packed to bf16, dK^T += Q~^T dX.
template <int D>
__device__ inline void kv_phase1_dv(const u32x4* T, u32x4* pl, const bf16x8 (&kreg)[D / 16], u32x4 (&pk)[4],
                                    float c, int hf, int l32, int lane) {
  constexpr int KSTEPS = BwdTile<D>::KSTEPS, CH = BwdTile<D>::CH;
  const u32x4* qcl = T + hf * KTILE + l32;
  const float* stl = reinterpret_cast<const float*>(T + 4 * CH);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) s = mfma32(as_bf16x8(qcl[2 * KTILE * ks + 32 * qb]), kreg[ks], s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 l4 = *reinterpret_cast<const float4*>(stl + 32 * qb + 8 * g + 4 * hf);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g], c, -l4.x));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 1], c, -l4.y));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 2], c, -l4.z));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + 3], c, -l4.w));
      const int kk = 2 * qb + (g >> 1), slot = 2 * (g & 1);
      pk[kk][slot] = pack_bf16x2(p0, p1);
      pk[kk][slot + 1] = pack_bf16x2(p2, p3);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pl[64 * kk + lane] = pk[kk];
}

template <int D>
__device__ inline void kv_phase1_dk(const u32x4* T, const bf16x8 (&vreg)[D / 16], f32x16 (&dp)[2], int hf,
                                    int l32) {
  constexpr int KSTEPS = BwdTile<D>::KSTEPS, CH = BwdTile<D>::CH;
  const u32x4* ocl = T + CH + hf * KTILE + l32;
  dp[0] = dp[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dp[qb] = mfma32(as_bf16x8(ocl[2 * KTILE * ks + 32 * qb]), vreg[ks], dp[qb]);
  }
}

template <int D>
__device__ inline void kv_phase2_dv(const u32x4* T, const u32x4 (&pk)[4], f32x16 (&acc)[D / 32], int hf, int l32) {
  constexpr int CH = BwdTile<D>::CH, DBLK = BwdTile<D>::DBLK;
  const u32x4* otl = T + 3 * CH + hf * D + l32;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 p8 = as_bf16x8(pk[ks]);
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] = mfma32(as_bf16x8(otl[2 * D * ks + 32 * b]), p8, acc[b]);
  }
}

template <int D>
__device__ inline void kv_phase2_dk(const u32x4* T, const u32x4* pl, const f32x16 (&dp)[2], f32x16 (&acc)[D / 32],
                                    int hf, int l32, int lane) {
  constexpr int CH = BwdTile<D>::CH, DBLK = BwdTile<D>::DBLK;
  const u32x4* qtl = T + 2 * CH + hf * D + l32;
  const float* stl = reinterpret_cast<const float*>(T + 4 * CH);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int qb = ks >> 1;
    const u32x4 p = pl[64 * ks + lane];
    uint32_t x[4];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * (ks & 1) + gg;
      const float4 d4 = *reinterpret_cast<const float4*>(stl + KTILE + 32 * qb + 8 * g + 4 * hf);
      const uint32_t w0 = p[2 * gg], w1 = p[2 * gg + 1];
      x[2 * gg] = pack_bf16x2(__uint_as_float(w0 << 16) * (dp[qb][4 * g] - d4.x),
                              __uint_as_float(w0 & 0xFFFF0000u) * (dp[qb][4 * g + 1] - d4.y));
      x[2 * gg + 1] = pack_bf16x2(__uint_as_float(w1 << 16) * (dp[qb][4 * g + 2] - d4.z),
                                  __uint_as_float(w1 & 0xFFFF0000u) * (dp[qb][4 * g + 3] - d4.w));
    }
    const bf16x8 x8 = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], x[2], x[3]});
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] = mfma32(as_bf16x8(qtl[2 * D * ks + 32 * b]), x8, acc[b]);
  }
}

// Position of a sample token for the epilogue rotations.
struct TokPos {
  int32_t row, col, frame;
};
template <bool R3>
__device__ inline TokPos token_pos(int32_t u, int32_t seg, const BwdArgs& a) {
  TokPos p{0, 0, 0};
  if constexpr (R3) token_position3(u, a.text_len[seg], a.grid_hw[2 * seg], a.grid_hw[2 * seg + 1], p.row, p.col, p.frame);
  else token_position(u, a.text_len[seg], a.grid_hw[2 * seg + 1], p.row, p.col);
  return p;
}

// Undo the rotation of four consecutive channels ch0 .. ch0+3 (two pairs) at
// position p and scale: (x0, x1) -> (x0 c + x1 s, -x0 s + x1 c) * scale.
template <int D, bool R3>
__device__ inline uint2 unrotate4(const float (&x)[4], int ch0, const TokPos& p, float scale, const BwdArgs& a) {
  float y[4];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int d = ch0 + 2 * pp;
    float2 r;
    if constexpr (R3) {
      r = rope3_cs(a.r3, D, d / 2, p.row, p.col, p.frame);
    } else {
      const bool first_half = d < D / 2;
      const int j = first_half ? d / 2 : (d - D / 2) / 2;
      r = a.cs[(first_half ? p.row : p.col) * (D / 4) + j];
    }
    const float x0 = x[2 * pp], x1 = x[2 * pp + 1];
    y[2 * pp] = (x0 * r.x + x1 * r.y) * scale;
    y[2 * pp + 1] = (x1 * r.x - x0 * r.y) * scale;
  }
  uint2 o;
  o.x = pack_bf16x2(y[0], y[1]);
  o.y = pack_bf16x2(y[2], y[3]);
  return o;
}

// Split of the dK/dV kernel's poorly filled last round (the plan of the
// forward, over units = KV_SPLIT x tiles x heads key blocks, pieces over query
// ranges): the same in every workgroup of both kernels. The last tile is the
// shortest sample's.
__device__ inline SplitPlan kv_plan(const BwdArgs& a, const WsHeader* hdr) {
  const int2 last = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[hdr->n_tiles - 1];
  const int32_t Ls = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[last.x];
  return split_plan(int64_t(KV_SPLIT) * hdr->n_tiles * a.heads, a.ncu, (Ls + KTILE - 1) / KTILE,
                    SPLIT_MIN_SAVED_BWD);
}

// The dQ kernel's plan: units = (256-query tile, head), split over key ranges
// when the last round fills the device poorly, with the forward's threshold
// (SPLIT_MIN_SAVED key tiles of the shortest unit).
__device__ inline SplitPlan q_plan(const BwdArgs& a, const WsHeader* hdr) {
  const int2 last = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[hdr->n_tiles - 1];
  const int32_t Ls = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[last.x];
  return split_plan(int64_t(hdr->n_tiles) * a.heads, a.ncu_q, (Ls + KTILE - 1) / KTILE);
}

template <int D, bool R3>
__global__ void __launch_bounds__(64 * KV_WAVES, 2) bwd_kv_kernel(BwdArgs a) {
  constexpr int CH = BwdTile<D>::CH, KSTEPS = BwdTile<D>::KSTEPS, DBLK = BwdTile<D>::DBLK;
  constexpr int SET = 4 * CH + 2 * KTILE / 4;  // chunks of one LDS tile set (4 tiles + stats)
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t heads = a.heads;
  if (hdr->flag != FLAG_OK) return;
  // Unit (key block, head) of this workgroup: a whole unit, or piece `part`
  // of a unit of the split last round (its query tiles [qt0, qt1)).
  const SplitPlan plan = kv_plan(a, hdr);
  int unit = int(blockIdx.x), part = -1;
  if (unit >= plan.n_full) {
    const int piece = unit - plan.n_full;
    if (piece >= plan.n_tail * plan.parts) return;
    unit = plan.n_full + piece / plan.parts;
    part = piece % plan.parts;
  }
  const int h = unit % heads;
  const int rest = unit / heads;
  const int tile = rest / KV_SPLIT;
  const int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x, k0 = td.y + KV_KEYS * (rest % KV_SPLIT);
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  if (k0 >= L) return;
  const int nqt_all = (L + KTILE - 1) / KTILE;
  int qt0 = 0, qt1 = nqt_all;
  if (part >= 0) {
    qt0 = part * nqt_all / plan.parts;
    qt1 = (part + 1) * nqt_all / plan.parts;
    if (qt0 == qt1) return;  // empty piece: the merge skips it
  }
  const int32_t pb = reinterpret_cast<const int32_t*>(a.ws + a.off_pcu)[seg];
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Waves [0, KV_GROUPS) accumulate dV, the others dK, of the same key groups.
  const bool dv_wave = wave < KV_GROUPS;
  const int group = dv_wave ? wave : wave - KV_GROUPS;
  const int64_t tile0 = (int64_t(h) * a.rows + pb) / KTILE;  // first KTILE tile of this (sample, head)

  // This lane's key as the B operand of S = Q~ K~^T and dP = dO V^T: key
  // k0 + 32 group + l32, channels 16ks + 8hf .. +7, read from the chunk-major
  // K~ and V tiles. Keys past the sample are zero (never stored).
  const int32_t key = k0 + 32 * group + l32;
  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
  {
    const int64_t r = tile0 * KTILE + key;
    const u32x4* kp = reinterpret_cast<const u32x4*>(a.kc) + (r / KTILE) * CH + hf * KTILE + (r % KTILE);
    const u32x4* vp = reinterpret_cast<const u32x4*>(a.vc) + (r / KTILE) * CH + hf * KTILE + (r % KTILE);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kreg[ks] = key < L && dv_wave ? as_bf16x8(kp[2 * KTILE * ks]) : bf16x8{};
      vreg[ks] = key < L && !dv_wave ? as_bf16x8(vp[2 * KTILE * ks]) : bf16x8{};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): later waits cover tile copies only
  __builtin_amdgcn_sched_barrier(0);

  __shared__ u32x4 sets[2 * SET];
  __shared__ u32x4 pex[KV_GROUPS * 4 * 64];  // P exchange: 4 KB per key group
  u32x4* pl = pex + group * 4 * 64;
  const u32x4* qcg = reinterpret_cast<const u32x4*>(a.qc) + tile0 * CH;
  const u32x4* ocg = reinterpret_cast<const u32x4*>(a.oc) + tile0 * CH;
  const u32x4* qtg = reinterpret_cast<const u32x4*>(a.qt) + tile0 * CH;
  const u32x4* otg = reinterpret_cast<const u32x4*>(a.ot) + tile0 * CH;
  const u32x4* stg = reinterpret_cast<const u32x4*>(a.st) + tile0 * (2 * KTILE / 4);
  auto load_set = [&](int j, u32x4* dst) {
    copy_to_lds<CH, KV_WAVES>(qcg + int64_t(j) * CH, dst, wave, lane);
    copy_to_lds<CH, KV_WAVES>(ocg + int64_t(j) * CH, dst + CH, wave, lane);
    copy_to_lds<CH, KV_WAVES>(qtg + int64_t(j) * CH, dst + 2 * CH, wave, lane);
    copy_to_lds<CH, KV_WAVES>(otg + int64_t(j) * CH, dst + 3 * CH, wave, lane);
    if (wave == 0 && lane < 2 * KTILE / 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(stg + int64_t(j) * (2 * KTILE / 4), 2 * KTILE * 4),
                                               (lds_ptr_t)(dst + 4 * CH), 16, lane * 16, 0, 0, 0);
  };

  f32x16 acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16{};
  const int nqt = qt1 - qt0;
  load_set(qt0, sets);
  wait_vm_and_sync();
  u32x4 pk[4];     // dV waves: this step's P (bf16), as the B operand of its four k-steps
  f32x16 dp[2];    // dK waves: this step's dP, two 32-query halves
  for (int jj = 0; jj < nqt; ++jj) {
    const u32x4* cur = sets + (jj & 1) * SET;
    if (dv_wave) kv_phase1_dv<D>(cur, pl, kreg, pk, a.c_log2, hf, l32, lane);
    else kv_phase1_dk<D>(cur, vreg, dp, hf, l32);
    // The next step's tiles go to the other set (last read in the previous
    // step). Issued after this step's first phase, not before it, so that
    // the 64 copy instructions do not hold back the start of the MFMAs.
    if (jj + 1 < nqt) load_set(qt0 + jj + 1, sets + ((jj + 1) & 1) * SET);
    __syncthreads();  // P of this step is in pl
    if (dv_wave) kv_phase2_dv<D>(cur, pk, acc, hf, l32);
    else kv_phase2_dk<D>(cur, pl, dp, acc, hf, l32, lane);
    wait_vm_and_sync();  // next tile set landed; pl and the current set may be overwritten
  }

  // Epilogue: entry e of block b is channel 32b + 8(e/4) + 4hf + e%4 of this lane's key.
  if (part >= 0) {
    // Piece of a split unit: fp32 dV (dV waves) or dK before the inverse
    // rotation (dK waves) of this lane's key into the piece's slot.
    float* slot = a.part + int64_t(blockIdx.x - plan.n_full) * 2 * KV_KEYS * D + (dv_wave ? 0 : KV_KEYS * D) +
                  int64_t(32 * group + l32) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(slot + 32 * b + 8 * g + 4 * hf) =
            make_float4(acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]);
    }
    return;
  }
  if (key < L) {
    const TokPos pos = token_pos<R3>(key, seg, a);
    const int64_t off = (int64_t(cb + key) * heads + h) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * b + 8 * g + 4 * hf;
        if (dv_wave) {
          uint2 o;
          o.x = pack_bf16x2(acc[b][4 * g], acc[b][4 * g + 1]);
          o.y = pack_bf16x2(acc[b][4 * g + 2], acc[b][4 * g + 3]);
          *reinterpret_cast<uint2*>(a.dv + off + ch) = o;
        } else {
          const float xk[4] = {acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
          *reinterpret_cast<uint2*>(a.dk + off + ch) = unrotate4<D, R3>(xk, ch, pos, a.scale, a);
        }
      }
    }
  }
}

// Merge of the pieces of split dK/dV unit u of the tail: per key and 4
// channels, the pieces' dV and dK sums in piece order (deterministic), then the
// epilogue of the whole-unit path (dV to bf16; dK inverse-rotated, scaled, to
// bf16). Run by extra workgroups of the dQ kernel, which is launched after the
// dK/dV kernel has finished, so every piece is complete; they take CUs that
// the dQ kernel's own last round leaves idle, and no launch is added.
template <int D, bool R3>
__device__ inline void kv_merge_unit(const BwdArgs& a, int u, int tid, int nthreads) {
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t heads = a.heads;
  const SplitPlan plan = kv_plan(a, hdr);
  if (u >= plan.n_tail) return;
  const int unit = plan.n_full + u;
  const int h = unit % heads;
  const int rest = unit / heads;
  const int tile = rest / KV_SPLIT;
  const int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x, k0 = td.y + KV_KEYS * (rest % KV_SPLIT);
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  if (k0 >= L) return;
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int nqt = (L + KTILE - 1) / KTILE;
  const int S = plan.parts;
  constexpr int64_t SLOT = int64_t(2) * KV_KEYS * D;
  const float* base = a.part + int64_t(u) * S * SLOT;
  for (int item = tid; item < KV_KEYS * D / 4; item += nthreads) {
    const int key = item / (D / 4), ch0 = 4 * (item % (D / 4));
    if (k0 + key >= L) break;  // items are key-major: the rest lie past the sample too
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f), sk = sv;
    for (int p = 0; p < S; ++p) {
      if ((p + 1) * nqt / S == p * nqt / S) continue;  // empty piece (never written)
      const float* sl = base + p * SLOT + int64_t(key) * D + ch0;
      const float4 x = *reinterpret_cast<const float4*>(sl);
      const float4 y = *reinterpret_cast<const float4*>(sl + KV_KEYS * D);
      sv.x += x.x; sv.y += x.y; sv.z += x.z; sv.w += x.w;
      sk.x += y.x; sk.y += y.y; sk.z += y.z; sk.w += y.w;
    }
    const int64_t off = (int64_t(cb + k0 + key) * heads + h) * D + ch0;
    uint2 o;
    o.x = pack_bf16x2(sv.x, sv.y);
    o.y = pack_bf16x2(sv.z, sv.w);
    *reinterpret_cast<uint2*>(a.dv + off) = o;
    const float xk[4] = {sk.x, sk.y, sk.z, sk.w};
    *reinterpret_cast<uint2*>(a.dk + off) = unrotate4<D, R3>(xk, ch0, token_pos<R3>(k0 + key, seg, a), a.scale, a);
  }
}

// ---------------------------------------------------------------- dQ

// One 64-key tile for one wave's 32 queries. T: LDS tile set [kc | vc | kt].
template <int D, bool MASKED>
__device__ inline void q_step(const u32x4* T, const bf16x8 (&qreg)[D / 16], const bf16x8 (&oreg)[D / 16],
                              f32x16 (&acc)[D / 32], float c, float lse2, float dsum, int kbase, int L,
                              int hf, int l32) {
  constexpr int CH = BwdTile<D>::CH, KSTEPS = BwdTile<D>::KSTEPS, DBLK = BwdTile<D>::DBLK;
  const u32x4* kcl = T + hf * KTILE + l32;
  const u32x4* vcl = T + CH + hf * KTILE + l32;
  const u32x4* ktl = T + 2 * CH + hf * D + l32;
  // S^T and dP^T (keys x queries), two 32-key blocks; lane = query l32,
  // entry e of block kb = key 32kb + 8(e/4) + 4hf + e%4.
  f32x16 s[2] = {}, dp[2] = {};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = mfma32(as_bf16x8(kcl[2 * KTILE * ks + 32 * kb]), qreg[ks], s[kb]);
      dp[kb] = mfma32(as_bf16x8(vcl[2 * KTILE * ks + 32 * kb]), oreg[ks], dp[kb]);
    }
  }
  uint32_t pd[4][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c, -lse2));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + 1], c, -lse2));
      if constexpr (MASKED) {
        const int key = kbase + 32 * kb + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (key >= L) p0 = 0.f;
        if (key + 1 >= L) p1 = 0.f;
      }
      pd[2 * kb + (e >> 3)][(e & 7) >> 1] = pack_bf16x2(p0 * (dp[kb][e] - dsum), p1 * (dp[kb][e + 1] - dsum));
    }
  }
  // dQ^T (channels x queries) += K~^T dX^T
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 x8 = __builtin_bit_cast(bf16x8, u32x4{pd[ks][0], pd[ks][1], pd[ks][2], pd[ks][3]});
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] = mfma32(as_bf16x8(ktl[2 * D * ks + 32 * b]), x8, acc[b]);
  }
}

template <int D, bool R3>
__global__ void __launch_bounds__(64 * Q_WAVES, 2) bwd_q_kernel(BwdArgs a) {
  constexpr int CH = BwdTile<D>::CH, KSTEPS = BwdTile<D>::KSTEPS, DBLK = BwdTile<D>::DBLK;
  constexpr int SET = 3 * CH;
  if (int64_t(blockIdx.x) >= a.dq_units) {  // workgroups past the dQ grid merge split dK/dV units
    kv_merge_unit<D, R3>(a, int(int64_t(blockIdx.x) - a.dq_units), int(threadIdx.x), 64 * Q_WAVES);
    return;
  }
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t heads = a.heads;
  if (hdr->flag != FLAG_OK) return;
  // A whole unit, or piece `part` of a unit of the split last round (its key
  // tiles [kt0, kt1)); workgroups past the plan return at once.
  const SplitPlan plan = q_plan(a, hdr);
  int unit = int(blockIdx.x), part = -1;
  if (unit >= plan.n_full) {
    const int piece = unit - plan.n_full;
    if (piece >= plan.n_tail * plan.parts) return;
    unit = plan.n_full + piece / plan.parts;
    part = piece % plan.parts;
  }
  int tile = unit / heads;
  int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x;
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  if (part < 0) {
    unit = xcd_unit(unit, heads, tile, td.y, L, plan.n_full);
    tile = unit / heads;
    td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  }
  const int h = unit % heads;
  const int32_t qs = td.y;
  const int32_t pb = reinterpret_cast<const int32_t*>(a.ws + a.off_pcu)[seg];
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int nkt_all = (L + KTILE - 1) / KTILE;
  int kt0 = 0, kt1 = nkt_all;
  if (part >= 0) {
    kt0 = part * nkt_all / plan.parts;
    kt1 = (part + 1) * nkt_all / plan.parts;
    if (kt0 == kt1) return;  // empty piece of a short unit: the merge skips it
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int64_t tile0 = (int64_t(h) * a.rows + pb) / KTILE;

  // This lane's query (rotated) and its dO row as B operands, plus its LSE
  // and D. Query rows past the sample are never stored; they get P = 0.
  const int32_t qrel = qs + 32 * wave + l32;
  const int64_t r = tile0 * KTILE + qrel;  // inside the padded buffer (its slack covers a whole tile)
  bf16x8 qreg[KSTEPS], oreg[KSTEPS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.qc) + (r / KTILE) * CH + hf * KTILE + (r % KTILE);
    const u32x4* op = reinterpret_cast<const u32x4*>(a.oc) + (r / KTILE) * CH + hf * KTILE + (r % KTILE);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qreg[ks] = as_bf16x8(qp[2 * KTILE * ks]);
      oreg[ks] = as_bf16x8(op[2 * KTILE * ks]);
    }
  }
  const float* stp = a.st + (r / KTILE) * (2 * KTILE) + (r % KTILE);
  const float lse2 = qrel < L ? stp[0] : INFINITY;
  const float dsum = qrel < L ? stp[KTILE] : 0.f;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);

  __shared__ u32x4 sets[2 * SET];
  const u32x4* kcg = reinterpret_cast<const u32x4*>(a.kc) + tile0 * CH;
  const u32x4* vcg = reinterpret_cast<const u32x4*>(a.vc) + tile0 * CH;
  const u32x4* ktg = reinterpret_cast<const u32x4*>(a.kt) + tile0 * CH;
  auto load_set = [&](int j, u32x4* dst) {
    copy_to_lds<CH, Q_WAVES>(kcg + int64_t(j) * CH, dst, wave, lane);
    copy_to_lds<CH, Q_WAVES>(vcg + int64_t(j) * CH, dst + CH, wave, lane);
    copy_to_lds<CH, Q_WAVES>(ktg + int64_t(j) * CH, dst + 2 * CH, wave, lane);
  };

  f32x16 acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16{};
  const int nkt = kt1 - kt0;
  load_set(kt0, sets);
  wait_vm_and_sync();
  for (int jj = 0; jj + 1 < nkt; ++jj) {
    load_set(kt0 + jj + 1, sets + ((jj + 1) & 1) * SET);
    q_step<D, false>(sets + (jj & 1) * SET, qreg, oreg, acc, a.c_log2, lse2, dsum, KTILE * (kt0 + jj), L, hf, l32);
    wait_vm_and_sync();
  }
  // The sample's last key tile carries the key mask.
  if (kt1 == nkt_all)
    q_step<D, true>(sets + ((nkt - 1) & 1) * SET, qreg, oreg, acc, a.c_log2, lse2, dsum, KTILE * (kt1 - 1), L,
                    hf, l32);
  else
    q_step<D, false>(sets + ((nkt - 1) & 1) * SET, qreg, oreg, acc, a.c_log2, lse2, dsum, KTILE * (kt1 - 1), L,
                     hf, l32);

  if (part >= 0) {
    // Piece of a split unit: the fp32 partial dQ (before the inverse rotation)
    // of its 256 rows into its slot, for bwd_q_merge_kernel.
    float* slot = a.qpart + int64_t(blockIdx.x - plan.n_full) * QTILE * D + int64_t(32 * wave + l32) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(slot + 32 * b + 8 * g + 4 * hf) =
            make_float4(acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]);
    }
    return;
  }
  if (qrel < L) {
    const TokPos pos = token_pos<R3>(qrel, seg, a);
    const int64_t off = (int64_t(cb + qrel) * heads + h) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * b + 8 * g + 4 * hf;
        const float x[4] = {acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
        *reinterpret_cast<uint2*>(a.dq + off + ch) = unrotate4<D, R3>(x, ch, pos, a.scale, a);
      }
    }
  }
}

// Merge of split dQ units: one workgroup per split unit; each row's channel
// quad is summed over the unit's non-empty pieces in piece order, then turned
// back (inverse rotation), scaled and rounded like a whole unit's epilogue.
template <int D, bool R3>
__global__ void __launch_bounds__(256) bwd_q_merge_kernel(BwdArgs a) {
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const SplitPlan plan = q_plan(a, hdr);
  const int u = int(blockIdx.x);
  if (u >= plan.n_tail) return;
  const int32_t heads = a.heads;
  const int unit = plan.n_full + u;
  const int h = unit % heads;
  const int tile = unit / heads;
  const int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x, qs = td.y;
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int nkt_all = (L + KTILE - 1) / KTILE;
  constexpr int QUADS = D / 4;  // channel quads per row
  const float* base = a.qpart + int64_t(u) * plan.parts * QTILE * D;
  for (int item = int(threadIdx.x); item < QTILE * QUADS; item += 256) {
    const int row = item / QUADS, c4 = item % QUADS;
    const int32_t qrel = qs + row;
    if (qrel >= L) continue;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < plan.parts; ++p) {
      if (p * nkt_all / plan.parts == (p + 1) * nkt_all / plan.parts) continue;  // empty piece
      const float4 x = *reinterpret_cast<const float4*>(base + int64_t(p) * QTILE * D + int64_t(row) * D + 4 * c4);
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const float xs[4] = {sum.x, sum.y, sum.z, sum.w};
    *reinterpret_cast<uint2*>(a.dq + (int64_t(cb + qrel) * heads + h) * D + 4 * c4) =
        unrotate4<D, R3>(xs, 4 * c4, token_pos<R3>(qrel, seg, a), a.scale, a);
  }
}

// ---------------------------------------------------------------- launch

template <int D, bool R3>
static hipError_t launch_bwd_t(const BwdArgs& a, const BwdLayout& l, hipStream_t s, hipEvent_t const* ev) {
  hipError_t e;
  hipLaunchKernelGGL((bwd_pack_kernel<D, R3>), dim3(unsigned(l.m.rows / KTILE), unsigned(a.heads)), dim3(256), 0,
                     s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  // Whole units, then up to PART_SLOTS pieces of split units (workgroups past
  // the plan return at once).
  hipLaunchKernelGGL((bwd_kv_kernel<D, R3>),
                     dim3(unsigned(KV_SPLIT * l.m.n_tiles * a.heads + (a.ncu > 0 ? PART_SLOTS : 0))),
                     dim3(64 * KV_WAVES), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return e;
  // The dQ grid (whole units, then up to PART_SLOTS pieces of split units),
  // then (when the dK/dV kernel may have split) one workgroup per possible
  // split dK/dV unit to merge it; then the merge of split dQ units.
  hipLaunchKernelGGL((bwd_q_kernel<D, R3>), dim3(unsigned(a.dq_units + (a.ncu > 0 ? PART_SLOTS / 2 : 0))),
                     dim3(64 * Q_WAVES), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.ncu_q > 0) hipLaunchKernelGGL((bwd_q_merge_kernel<D, R3>), dim3(PART_SLOTS / 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* grid_hw, const int32_t* text_len,
                           const float2* cs, const Rope3* r3, char* ws, const BwdLayout& l, void* dq, void* dk,
                           void* dv, int64_t tokens, int32_t heads, int32_t head_dim, float scale, int32_t ncu,
                           int32_t ncu_q, hipStream_t s, hipEvent_t const* ev) {
  BwdArgs a;
  a.ws = ws;
  a.off_len = l.m.off_len;
  a.off_cu = l.m.off_cu;
  a.off_pcu = l.m.off_pcu;
  a.off_tiles = l.m.off_tiles;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.grid_hw = grid_hw;
  a.text_len = text_len;
  a.cs = cs;
  a.r3 = r3 ? *r3 : Rope3{nullptr, 0, 0};
  a.qc = reinterpret_cast<uint16_t*>(ws + l.off_qc);
  a.qt = reinterpret_cast<uint16_t*>(ws + l.off_qt);
  a.oc = reinterpret_cast<uint16_t*>(ws + l.off_oc);
  a.ot = reinterpret_cast<uint16_t*>(ws + l.off_ot);
  a.kc = reinterpret_cast<uint16_t*>(ws + l.off_kc);
  a.kt = reinterpret_cast<uint16_t*>(ws + l.off_kt);
  a.vc = reinterpret_cast<uint16_t*>(ws + l.off_vc);
  a.st = reinterpret_cast<float*>(ws + l.off_st);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.heads = heads;
  a.rows = l.m.rows;
  a.tokens = tokens;
  a.c_log2 = scale * LOG2E;
  a.scale = scale;
  a.part = reinterpret_cast<float*>(ws + l.off_part);
  a.qpart = reinterpret_cast<float*>(ws + l.off_qpart);
  a.ncu = ncu;
  a.ncu_q = ncu_q;
  a.dq_units = l.m.n_tiles * heads + (ncu_q > 0 ? PART_SLOTS : 0);
  if (r3) return head_dim == 128 ? launch_bwd_t<128, true>(a, l, s, ev) : launch_bwd_t<64, true>(a, l, s, ev);
  return head_dim == 128 ? launch_bwd_t<128, false>(a, l, s, ev) : launch_bwd_t<64, false>(a, l, s, ev);
}

}  // namespace mf
