// Packed joint attention forward on gfx950.
//
// Operation: for every sample i and head h, O = softmax(Q~ K~^T / sqrt(d)) V
// over the sample's own L_i tokens only (Mage-Flow tech report, NR-MMDiT
// section: per-sample cumulative offsets restrict attention to each sample;
// mageflow.net architecture page, sections 2 and 8: text and image tokens in
// one bidirectional sequence). Q~, K~ are the 2D-RoPE-rotated queries and
// keys; K~ (and V~^T) are written by the prologue into the padded workspace layout, where every
// sample starts on a KTILE boundary; query tiles are sample-relative, so a
// workgroup only ever visits the key tiles of its own sample and the
// cross-sample blocks of the packed score matrix are never touched.
//
// bf16 kernel (d = 64 or 128), one workgroup = QTILE / 32 waves = QTILE queries
// (the queries are read from the caller's q and rotated while loading)
// of one (sample, head), each wave owning 32 query rows:
//   S^T (64 keys x 32 queries) = K~ tile (LDS) x Q~^T (registers), on
//       v_mfma_f32_32x32x16_bf16 with fp32 accumulation. In this orientation
//       every lane holds one query row: 32 of the 64 keys in registers, the
//       other 32 in lane ^ 32, so row max / sum need one cross-half exchange.
//   online softmax in the exp2 domain (scale * log2(e) folded into one FMA),
//       running max m, per-lane partial row sums (combined once at the end),
//       accumulator rescale skipped when no row max moved;
//   O^T (d x 32 queries) += V~^T tile (LDS) x P^T (registers, bf16 RNE).
// K~ and V~^T tiles (KTILE x d each) are double-buffered in LDS: the global
// loads of tile j+1 are issued before the math of tile j and written to the
// other LDS buffer after it, one barrier per tile.
//
// f32 kernel: the same tiling of work with plain fp32 FMAs (no reduced
// precision anywhere); each query row is split over two lanes (channel halves).
#include <type_traits>

#include "mf_common.h"
#include "mfma_util.h"
#include "rope_math.h"

namespace mf {

struct AttnArgs {
  const char* ws;
  int64_t off_len, off_cu, off_pcu, off_tiles;
  const void* q;            // caller's queries [T][heads][d] (bf16 kernel rotates them on load)
  const int32_t* grid_hw;   // caller's (h, w) per sample
  const int32_t* text_len;  // caller's prompt length per sample
  const float2* cs;         // cos/sin table [ROPE_PMAX][d/4]
  Rope3 r3;                 // frame-aware RoPE of editing samples (R3 kernels)
  const void* qw;           // rotated queries in the workspace (f32 kernel)
  const void* kw;
  const void* vw;
  void* out;
  float* lse;        // optional [heads][tokens] natural-log row sum-exp of the scaled scores
  float* part;       // partial results of split units (bf16 path), PART_SLOTS slots
  int32_t ncu;       // compute units for the split plan (0: never split)
  int64_t tokens;
  int32_t heads;
  int64_t rows;      // padded rows per head in the workspace
  float c_log2;      // softmax scale * log2(e)
};

// The split plan of this call (same in every workgroup of every kernel):
// units = tiles x heads, the shortest unit is the last tile's.
__device__ inline SplitPlan call_plan(const AttnArgs& a, const WsHeader* hdr) {
  const int2 last = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[hdr->n_tiles - 1];
  const int32_t Ls = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[last.x];
  return split_plan(int64_t(hdr->n_tiles) * a.heads, a.ncu, (Ls + KTILE - 1) / KTILE);
}

// Copies one chunk-major tile (CHUNKS 16-byte chunks) from the workspace into
// LDS with direct-to-LDS loads spread over the workgroup's waves.
template <int CHUNKS>
__device__ inline void tile_to_lds(const u32x4* __restrict__ src, u32x4* dst, int wave, int lane) {
  copy_to_lds<CHUNKS, ATTN_WAVES>(src, dst, wave, lane);
}

__device__ inline void wait_tile_and_sync() { wait_vm_and_sync(); }

template <int D>
struct Bf16Tile {
  static constexpr int CHUNKS = KTILE * D / 8;  // 16-byte chunks per K~ (or V~^T) tile
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps of the score product
  static constexpr int DBLK = D / 32;           // 32-channel blocks of the output
};

// One 64-key tile of one wave's 32 query rows: S^T = K~ Q~^T, online softmax,
// O^T += V~^T P^T. kt / vt point at the chunk-major K~ and V~^T tiles in LDS.
template <int D, bool MASKED>
__device__ inline void attend_tile(const u32x4* kt, const u32x4* vt, const bf16x8 (&qreg)[D / 16],
                                   f32x16 (&acc)[D / 32], float& m, float& lsum, float c,
                                   int kbase_key, int L, int hf, int l32) {
  constexpr int KSTEPS = Bf16Tile<D>::KSTEPS;
  constexpr int DBLK = Bf16Tile<D>::DBLK;
  constexpr float REF_SLACK = 8.0f;
  // K~ chunk (c, n) sits at c * KTILE + n: lane (l32, hf) reads key n = l32 (+32)
  // and channel chunk 2*ks + hf, i.e. base + 2*KTILE*ks (+32).
  const u32x4* kl = kt + hf * KTILE + l32;
  // V~^T chunk (g, r) sits at g * D + r: lane reads channel r = 32*b + l32, key chunk 2*ks2 + hf.
  const u32x4* vl = vt + hf * D + l32;

  f32x16 s0 = {}, s1 = {};
  bf16x8 kb0[4], kb1[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kb0[ks] = __builtin_bit_cast(bf16x8, kl[2 * KTILE * ks]);
    kb1[ks] = __builtin_bit_cast(bf16x8, kl[2 * KTILE * ks + 32]);
  }
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const bf16x8 a0 = kb0[ks & 3], a1 = kb1[ks & 3];
    if (ks + 4 < KSTEPS) {
      kb0[ks & 3] = __builtin_bit_cast(bf16x8, kl[2 * KTILE * (ks + 4)]);
      kb1[ks & 3] = __builtin_bit_cast(bf16x8, kl[2 * KTILE * (ks + 4) + 32]);
    }
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
  }
  // V operands of the first two k-steps, read while the softmax runs.
  bf16x8 vb[2][DBLK];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
    for (int b = 0; b < DBLK; ++b) vb[k2][b] = __builtin_bit_cast(bf16x8, vl[2 * D * k2 + 32 * b]);
  }
  // Accumulator entry e holds key 8*(e/4) + 4*hf + e%4 of the tile (s1: +32).
  if constexpr (MASKED) {
    const int kb = kbase_key + 4 * hf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kb + 8 * (e >> 2) + (e & 3);
      if (key >= L) s0[e] = -INFINITY;
      if (key + 32 >= L) s1[e] = -INFINITY;
    }
  }
  // Row max: this lane's 32 keys, then the other 32 from lane ^ 32.
  float mx = __builtin_elementwise_maximum(s0[0], s1[0]);
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s0[e]), s1[e]);
  const float mt = halves_max(mx) * c;
  // The reference max only moves when a tile's max exceeds it by more than
  // REF_SLACK, so p = exp2(s*c - m) <= 2^REF_SLACK and the accumulator is
  // rescaled only on those tiles; numerator and denominator share m.
  const bool grow = mt > m + REF_SLACK;  // always true on the first tile (m = -inf)
  if (__any(grow)) {
    const float mnew = grow ? mt : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 on the first tile, 1 where unchanged
    lsum *= alpha;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] *= alpha;
    m = mnew;
  }
  const float nm = -m;
  uint32_t pk[4][4];  // P^T operand: k-step ks2 holds keys 16*ks2 + {4hf..4hf+3, 8+4hf..8+4hf+3}
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[e], c, nm));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[e + 1], c, nm));
    const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[e], c, nm));
    const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[e + 1], c, nm));
    pk[e >> 3][(e & 7) >> 1] = pack_bf16x2(p0, p1);
    pk[2 + (e >> 3)][(e & 7) >> 1] = pack_bf16x2(p2, p3);
  }
  // Row sum of the bf16 P actually multiplied into V (two keys per v_dot2).
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum = dot2_bf16_sum(pk[k2][i], lsum);
  }
  // O^T += V~^T x P^T
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    const bf16x8 pb8 = __builtin_bit_cast(bf16x8, u32x4{pk[ks2][0], pk[ks2][1], pk[ks2][2], pk[ks2][3]});
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const bf16x8 vv = vb[ks2 & 1][b];
      if (ks2 + 2 < 4) vb[ks2 & 1][b] = __builtin_bit_cast(bf16x8, vl[2 * D * (ks2 + 2) + 32 * b]);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb8, acc[b], 0, 0, 0);
    }
  }
}

template <int D, bool R3>
__global__ void __launch_bounds__(ATTN_THREADS, 2) attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int CHUNKS = Bf16Tile<D>::CHUNKS;
  constexpr int KSTEPS = Bf16Tile<D>::KSTEPS;
  constexpr int DBLK = Bf16Tile<D>::DBLK;

  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t heads = a.heads;
  if (hdr->flag != FLAG_OK) return;
  // Unit (query tile, head) of this workgroup: a whole unit, or piece `part`
  // of a unit of the split last round (its key tiles [kt0, kt1)).
  const SplitPlan plan = call_plan(a, hdr);
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
  const int64_t head_row0 = int64_t(h) * a.rows + pb;  // first padded row of this (sample, head)

  // Rotated query row of this lane as the B operand of S^T = K~ Q~^T: lane
  // holds query l32, channels 16*ks + 8*hf .. +7 for every k-step ks. The row
  // is read from the caller's q and rotated here (once per workgroup); rows
  // past the sample's end read its last token and are never stored.
  bf16x8 qreg[KSTEPS];
  {
    const int32_t u = min(qs + 32 * wave + l32, L - 1);
    int32_t row, col, frame = 0;
    if constexpr (R3) token_position3(u, a.text_len[seg], a.grid_hw[2 * seg], a.grid_hw[2 * seg + 1], row, col, frame);
    else token_position(u, a.text_len[seg], a.grid_hw[2 * seg + 1], row, col);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t(cb + u) * heads + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const Chunk<uint16_t> raw = *reinterpret_cast<const Chunk<uint16_t>*>(qrow + 16 * ks);
      if constexpr (R3)
        qreg[ks] = __builtin_bit_cast(bf16x8, rotate_chunk3<uint16_t, D>(raw, 16 * ks + 8 * hf, row, col, frame, a.r3));
      else
        qreg[ks] = __builtin_bit_cast(bf16x8, rotate_chunk<uint16_t, D>(raw, 16 * ks + 8 * hf, row, col, a.cs));
    }
  }
  // The tile copies share the in-order vector-memory counter with these
  // loads: finish Q first so later waits only cover tile copies.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);

  // Two LDS buffers, each one K~ tile and one V~^T tile (chunk-major, verbatim copies).
  __shared__ u32x4 kA[CHUNKS], vA[CHUNKS], kB[CHUNKS], vB[CHUNKS];
  // Key tiles [kt0, kt1) of the sample; the sample's last tile carries the key mask.
  const u32x4* kg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.kw) + head_row0 * D) + kt0 * CHUNKS;
  const u32x4* vg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.vw) + head_row0 * D) + kt0 * CHUNKS;
  const int nkt = kt1 - kt0;
  const int key0 = KTILE * kt0;
  const bool mask_last = kt1 == nkt_all;

  const float c = a.c_log2;
  float m = -INFINITY;  // reference row max (log2 units)
  float lsum = 0.f;     // this lane's partial row sum (its 32 keys of every tile)
  f32x16 acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16{};

  tile_to_lds<CHUNKS>(kg, kA, wave, lane);
  tile_to_lds<CHUNKS>(vg, vA, wave, lane);
  wait_tile_and_sync();
  // Tiles alternate between buffer A (even j) and B (odd j); the copy of tile
  // j+1 runs while tile j is processed. The last tile carries the key mask.
  int j = 0;
  for (; j + 2 < nkt; j += 2) {
    tile_to_lds<CHUNKS>(kg + (j + 1) * CHUNKS, kB, wave, lane);
    tile_to_lds<CHUNKS>(vg + (j + 1) * CHUNKS, vB, wave, lane);
    attend_tile<D, false>(kA, vA, qreg, acc, m, lsum, c, key0 + KTILE * j, L, hf, l32);
    wait_tile_and_sync();
    tile_to_lds<CHUNKS>(kg + (j + 2) * CHUNKS, kA, wave, lane);
    tile_to_lds<CHUNKS>(vg + (j + 2) * CHUNKS, vA, wave, lane);
    attend_tile<D, false>(kB, vB, qreg, acc, m, lsum, c, key0 + KTILE * (j + 1), L, hf, l32);
    wait_tile_and_sync();
  }
  if (j + 1 < nkt) {
    tile_to_lds<CHUNKS>(kg + (j + 1) * CHUNKS, kB, wave, lane);
    tile_to_lds<CHUNKS>(vg + (j + 1) * CHUNKS, vB, wave, lane);
    attend_tile<D, false>(kA, vA, qreg, acc, m, lsum, c, key0 + KTILE * j, L, hf, l32);
    wait_tile_and_sync();
    if (mask_last) attend_tile<D, true>(kB, vB, qreg, acc, m, lsum, c, key0 + KTILE * (j + 1), L, hf, l32);
    else attend_tile<D, false>(kB, vB, qreg, acc, m, lsum, c, key0 + KTILE * (j + 1), L, hf, l32);
  } else {
    if (mask_last) attend_tile<D, true>(kA, vA, qreg, acc, m, lsum, c, key0 + KTILE * j, L, hf, l32);
    else attend_tile<D, false>(kA, vA, qreg, acc, m, lsum, c, key0 + KTILE * j, L, hf, l32);
  }

  // Epilogue: O = acc / l. Accumulator entry e of block b holds channel
  // 32*b + 8*(e/4) + 4*hf + e%4 of query l32.
  lsum = halves_sum(lsum);
  if (part >= 0) {
    // Piece of a split unit: unnormalized accumulator, reference max and row
    // sum into its slot, for the merge kernel.
    const int r = 32 * wave + l32;
    float* slot = a.part + int64_t(blockIdx.x - plan.n_full) * QTILE * (D + 2);
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(slot + int64_t(r) * D + 32 * b + 8 * g + 4 * hf) =
            make_float4(acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]);
    }
    if (hf == 0) {
      slot[QTILE * D + r] = m;
      slot[QTILE * D + QTILE + r] = lsum;
    }
    return;
  }
  const float inv = 1.f / lsum;
  const int32_t qrel = qs + 32 * wave + l32;
  // log-sum-exp in natural-log units: p = 2^(s c - m) / lsum, so
  // ln sum_k e^(s_k * scale) = (m + log2 lsum) * ln 2.
  if (a.lse && qrel < L && hf == 0) a.lse[int64_t(h) * a.tokens + cb + qrel] = (m + log2f(lsum)) * 0.6931471805599453f;
  if (qrel < L) {
    uint16_t* orow = static_cast<uint16_t*>(a.out) + (int64_t(cb + qrel) * heads + h) * D;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v2;
        v2.x = pack_bf16x2(acc[b][4 * g] * inv, acc[b][4 * g + 1] * inv);
        v2.y = pack_bf16x2(acc[b][4 * g + 2] * inv, acc[b][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * b + 8 * g + 4 * hf) = v2;
      }
    }
  }
}

// Merge of the pieces of split units. Piece i of a unit holds, per query row,
// an accumulator and a row sum taken relative to its own reference max m_i;
// with M = max_i m_i and w_i = 2^(m_i - M) the row is
//   O = sum_i w_i acc_i / sum_i w_i l_i,   log-sum-exp = (M + log2 sum_i w_i l_i) ln 2,
// summed in piece order (deterministic). Each workgroup takes 64 rows of one
// split unit, each wave 16 rows: lanes 0-15 form the weights of one row each,
// then all lanes stream the rows' accumulators (D/64 channels per lane) with
// the weights broadcast from those lanes, every row's loads issued together.
constexpr int MERGE_ROWS = 64;  // rows per merge workgroup
template <int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnArgs a) {
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t heads = a.heads;
  const SplitPlan plan = call_plan(a, hdr);
  constexpr int BLOCKS = QTILE / MERGE_ROWS;
  const int u = int(blockIdx.x) / BLOCKS;
  if (u >= plan.n_tail) return;
  const int unit = plan.n_full + u;
  const int h = unit % heads, tile = unit / heads;
  const int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x, qs = td.y;
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = MERGE_ROWS * (int(blockIdx.x) % BLOCKS) + 16 * wave;  // this wave's first row
  if (qs + r0 >= L) return;
  const int nkt = (L + KTILE - 1) / KTILE;
  const int S = plan.parts;  // 2 to 4
  constexpr int CPL = D / 64;
  constexpr int64_t SLOT = int64_t(QTILE) * (D + 2);
  const float* slot0 = a.part + int64_t(u) * S * SLOT;
  // Weights of row r0 + lane (lanes 0-15); an empty piece (never written) weighs 0.
  float wgt[4] = {0.f, 0.f, 0.f, 0.f}, inv = 0.f;
  if (lane < 16) {
    const int r = r0 + lane;
    float mp[4], lp[4];
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool live = p < S && (p + 1) * nkt / S != p * nkt / S;
      mp[p] = live ? slot0[p * SLOT + QTILE * D + r] : -INFINITY;
      lp[p] = live ? slot0[p * SLOT + QTILE * D + QTILE + r] : 0.f;
      M = fmaxf(M, mp[p]);
    }
    float lsum = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      wgt[p] = lp[p] > 0.f ? __builtin_amdgcn_exp2f(mp[p] - M) : 0.f;
      lsum += wgt[p] * lp[p];
    }
    inv = 1.f / lsum;
    if (a.lse && qs + r < L) a.lse[int64_t(h) * a.tokens + cb + qs + r] = (M + log2f(lsum)) * 0.6931471805599453f;
  }
#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int r = r0 + rr;
    if (qs + r >= L) break;  // same for the whole wave
    float o[CPL] = {};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float w = __shfl(wgt[p], rr);
      if (w != 0.f) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[e] += w * slot0[p * SLOT + int64_t(r) * D + CPL * lane + e];
      }
    }
    const float ir = __shfl(inv, rr);
    uint16_t* orow = static_cast<uint16_t*>(a.out) + (int64_t(cb + qs + r) * heads + h) * D + CPL * lane;
    if constexpr (CPL == 2) *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(o[0] * ir, o[1] * ir);
    else orow[0] = uint16_t(pack_bf16x2(o[0] * ir, 0.f) & 0xFFFFu);
  }
}

// fp32 path: QTILE / 32 waves x 32 queries; lane = (query l32, channel half hf).
template <int D>
__global__ void __launch_bounds__(ATTN_THREADS) attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int HD = D / 2;
  constexpr int KT = 32;  // keys per LDS tile
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t heads = a.heads;
  const int h = int(blockIdx.x % unsigned(heads));
  const int tile = int(blockIdx.x / unsigned(heads));
  if (hdr->flag != FLAG_OK || tile >= hdr->n_tiles) return;
  const int2 td = reinterpret_cast<const int2*>(a.ws + a.off_tiles)[tile];
  const int32_t seg = td.x, qs = td.y;
  const int32_t L = reinterpret_cast<const int32_t*>(a.ws + a.off_len)[seg];
  const int32_t pb = reinterpret_cast<const int32_t*>(a.ws + a.off_pcu)[seg];
  const int32_t cb = reinterpret_cast<const int32_t*>(a.ws + a.off_cu)[seg];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int64_t head_row0 = int64_t(h) * a.rows + pb;
  const float* qw = static_cast<const float*>(a.qw);
  const float* kw = static_cast<const float*>(a.kw) + head_row0 * D;
  const float* vw = static_cast<const float*>(a.vw) + head_row0 * D;

  float qv[HD], acc[HD];
  const float* qrow = qw + (head_row0 + qs + 32 * wave + l32) * D + HD * hf;
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    qv[i] = qrow[i];
    acc[i] = 0.f;
  }
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const float c = a.c_log2;
  float m = -INFINITY, lsum = 0.f;
  const int nkt = (L + KT - 1) / KT;
  for (int j = 0; j < nkt; ++j) {
    __syncthreads();
    for (int x = tid; x < KT * D; x += ATTN_THREADS) {
      ks[x / D][x % D] = kw[int64_t(j) * KT * D + x];
      vs[x / D][x % D] = vw[int64_t(j) * KT * D + x];
    }
    __syncthreads();
    float s[KT];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < HD; ++i) part = __builtin_fmaf(qv[i], ks[kk][HD * hf + i], part);
      const float full = part + __shfl_xor(part, 32);
      s[kk] = (KT * j + kk < L) ? full * c : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2f(m - mnew);
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < HD; ++i) acc[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const float p = exp2f(s[kk] - mnew);
      lsum += p;
#pragma unroll
      for (int i = 0; i < HD; ++i) acc[i] = __builtin_fmaf(p, vs[kk][HD * hf + i], acc[i]);
    }
    m = mnew;
  }
  const int32_t qrel = qs + 32 * wave + l32;
  if (a.lse && qrel < L && hf == 0) a.lse[int64_t(h) * a.tokens + cb + qrel] = (m + log2f(lsum)) * 0.6931471805599453f;
  if (qrel < L) {
    float* orow = static_cast<float*>(a.out) + (int64_t(cb + qrel) * heads + h) * D + HD * hf;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < HD; ++i) orow[i] = acc[i] * inv;
  }
}

hipError_t launch_attn_fwd(char* ws, const WsLayout& l, const void* q, const int32_t* grid_hw,
                           const int32_t* text_len, const float2* cs, const Rope3* r3, void* out, float* lse,
                           int64_t tokens, int32_t heads, int32_t head_dim, bool bf16, float scale, int32_t ncu,
                           hipStream_t s) {
  AttnArgs a;
  a.ws = ws;
  a.q = q;
  a.grid_hw = grid_hw;
  a.text_len = text_len;
  a.cs = cs;
  a.r3 = r3 ? *r3 : Rope3{nullptr, 0, 0};
  a.off_len = l.off_len;
  a.off_cu = l.off_cu;
  a.off_pcu = l.off_pcu;
  a.off_tiles = l.off_tiles;
  a.qw = ws + l.off_q;
  a.kw = ws + l.off_k;
  a.vw = ws + l.off_v;
  a.out = out;
  a.lse = lse;
  a.part = reinterpret_cast<float*>(ws + l.off_part);
  a.ncu = bf16 ? ncu : 0;  // the fp32 path never splits
  a.tokens = tokens;
  a.heads = heads;
  a.rows = l.rows;
  a.c_log2 = scale * 1.4426950408889634f;
  // Whole units, then up to PART_SLOTS pieces of split units; workgroups past
  // the plan return at once.
  const dim3 grid(unsigned(l.n_tiles * heads + (a.ncu > 0 ? PART_SLOTS : 0)));
  if (bf16) {
    if (r3) {
      if (head_dim == 128) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), grid, dim3(ATTN_THREADS), 0, s, a);
      else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), grid, dim3(ATTN_THREADS), 0, s, a);
    } else {
      if (head_dim == 128) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), grid, dim3(ATTN_THREADS), 0, s, a);
      else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), grid, dim3(ATTN_THREADS), 0, s, a);
    }
  } else {
    if (head_dim == 128) hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(ATTN_THREADS), 0, s, a);
    else hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(ATTN_THREADS), 0, s, a);
  }
  if (a.ncu > 0) {
    // Split units: at most PART_SLOTS / 2 (two or more pieces each).
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid(unsigned(PART_SLOTS / 2 * (QTILE / MERGE_ROWS)));
    if (head_dim == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mf
