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
// of one (sample, head), each wave owning 32 query rows as two blocks of 16:
//   S^T (64 keys x 16 queries per block) = K~ tile (LDS) x Q~^T (registers),
//       on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; each K~ operand
//       read feeds the MFMAs of both blocks. In this orientation a lane holds
//       16 of the 64 scores of one query and the other 48 sit in lanes l ^ 16,
//       l ^ 32 and l ^ 48, so row max / sum need two lane swaps.
//   online softmax in the exp2 domain: the queries carry scale * log2(e)
//       (multiplied in as they are rotated) and the score accumulators start
//       from -m, the reference max, so the MFMAs produce s c - m and P is
//       exp2 of the accumulator with no per-score VALU arithmetic; the
//       reference moves only when a tile exceeds it by 2^8 (the accumulator
//       rescale is skipped otherwise); row sums of the bf16 P formed by MFMAs
//       against an all-ones operand;
//   O^T (d x 16 queries per block) += V~^T tile (LDS) x P^T (registers, bf16 RNE).
// Per key tile a wave has an MFMA phase (P.V of the previous tile, scores of
// this tile, LDS operands read ahead) and a VALU phase (softmax). The two
// waves sharing a SIMD are one phase apart (waves 0-3 and 4-7, a barrier
// after every phase), so one issues MFMAs while the other runs its softmax.
// K~ and V~^T tiles (KTILE x d each) are triple-buffered in LDS and copied
// there by direct-to-LDS loads two tiles ahead.
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
  const void* q;            // caller's queries (bf16 kernel rotates them on load)
  int64_t q_st, q_sh;       // their element strides (token, head)
  int64_t o_st, o_sh;       // element strides of out
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
  static constexpr int KSTEPS = D / 32;         // MFMA k-steps of the score product
  static constexpr int CBLK = D / 16;           // 16-channel blocks of the output
};

// Max / sum of a value over the four lanes l % 16 + 16 r (r = 0..3): rows r
// and r ^ 2 through v_permlane32_swap, then rows r and r ^ 1 through
// v_permlane16_swap (with both operands equal, the two results hold the value
// of the lane's row pair, so the combine needs no lane test).
__device__ inline float quad_max(float x) {
  x = halves_max(x);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float quad_sum(float x) {
  x = halves_sum(x);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS operand reads issued ahead of their MFMAs in an MFMA phase.
constexpr int PF_DEPTH = 6;

// MFMA phase of tile j for one wave's 32 query rows (two blocks of 16): with
// PV, O^T += V~^T P^T for tile j-1 (P^T in pk, V~^T tile vt), then, with SC,
// S^T = K~ Q~^T c - m for tile j (K~ tile kt; negm = -m as the accumulators'
// initial value) into s. Lane (g, l16) = (lane / 16,
// lane % 16) holds, for query 16 qb + l16, the scores of keys 16 kb + 4 g + i
// (i = 0..3) in s[kb][qb] and the output channels 16 cb + 4 g + i in
// acc[cb][qb]. Each 16-byte operand read from LDS feeds the MFMAs of both
// query blocks and is issued PF_DEPTH operands ahead of them (the order is
// pinned by scheduling fences): in this phase the wave's SIMD partner runs
// its softmax, so no other wave's MFMAs cover the LDS latency. The products
// are summed in the same order as a plain loop (k-steps ks = 0.. for S, key
// halves jj = 0, 1 for O).
template <int D, bool PV, bool SC>
__device__ __attribute__((always_inline)) inline void mfma_phase(const u32x4* kt, const u32x4* vt,
                                                                 const bf16x8 (&qreg)[2][D / 32],
                                                                 f32x4 (&acc)[D / 16][2], f32x4 (&s)[4][2],
                                                                 const u32x4 (&pk)[2][2], f32x4 (&lsv)[2],
                                                                 const f32x4 (&negm)[2], int g, int l16) {
  constexpr int CBLK = Bf16Tile<D>::CBLK;
  constexpr int NV = PV ? 2 * CBLK : 0;              // V~^T operands: key half jj, channel block cb
  constexpr int NK = SC ? 4 * Bf16Tile<D>::KSTEPS : 0;  // K~ operands: k-step ks, key block kb
  constexpr int N = NV + NK;
  // K~ chunk (c, n) sits at c * KTILE + n: lane reads key 16 kb + l16, channel
  // chunk 4 ks + g. V~^T chunk (k8, r) sits at k8 * D + r and holds, for
  // channel r, keys 32 (k8 / 4) + 4 (k8 % 4) + {0..3, 16..19}: lane reads
  // channel 16 cb + l16, key chunk 4 jj + g, the keys its own P^T operand carries.
  const u32x4* kl = kt + g * KTILE + l16;
  const u32x4* vl = vt + g * D + l16;
  auto operand = [&](int r) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, r < NV ? vl[4 * D * (r / CBLK) + 16 * (r % CBLK)]
                                             : kl[4 * KTILE * ((r - NV) / 4) + 16 * ((r - NV) % 4)]);
  };
  bf16x8 op[N];
#pragma unroll
  for (int r = 0; r < PF_DEPTH && r < N; ++r) op[r] = operand(r);
  if constexpr (SC) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = negm[0];
      s[kb][1] = negm[1];
    }
  }
  // Row sums of tile j-1's bf16 P (the values just multiplied into V~^T): the
  // same MFMA with an all-ones A operand sums P^T over the 32 keys of a k-step
  // into every entry of lsv[qb]. Four MFMAs per tile take the 16 v_dot2 of
  // per-lane sums out of the softmax phase, whose exponentials run slower
  // while the SIMD partner issues MFMAs. They read no LDS operand, so they go
  // first, while the first operand reads are in flight.
  if constexpr (PV) {
    typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
    const bf16x8v ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                          (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      lsv[0] = mfma16(__builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, pk[jj][0]), lsv[0]);
      lsv[1] = mfma16(__builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, pk[jj][1]), lsv[1]);
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + PF_DEPTH < N) op[i + PF_DEPTH] = operand(i + PF_DEPTH);
    __builtin_amdgcn_sched_barrier(0);
    if (i < NV) {
      const int jj = i / CBLK, cb = i % CBLK;
      acc[cb][0] = mfma16(op[i], __builtin_bit_cast(bf16x8, pk[jj][0]), acc[cb][0]);
      acc[cb][1] = mfma16(op[i], __builtin_bit_cast(bf16x8, pk[jj][1]), acc[cb][1]);
    } else {
      const int ks = (i - NV) / 4, kb = (i - NV) % 4;
      s[kb][0] = mfma16(op[i], qreg[0][ks], s[kb][0]);
      s[kb][1] = mfma16(op[i], qreg[1][ks], s[kb][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// VALU phase of tile j: key mask (MASKED: keys from kbase_key on at or past L),
// online softmax in the exp2 domain and the bf16 P^T operand. P^T of query
// block qb for keys 32 jj .. 32 jj + 31: k-slots 8 g .. +3 are keys
// 32 jj + 4 g + i, slots 8 g + 4 .. +7 keys 32 jj + 16 + 4 g + i, i.e.
// s[2 jj][qb] and s[2 jj + 1][qb] of this lane.
template <int D, bool MASKED>
__device__ __attribute__((always_inline)) inline void valu_phase(f32x4 (&s)[4][2], f32x4 (&acc)[D / 16][2],
                                                                 float (&m)[2], f32x4 (&lsv)[2], u32x4 (&pk)[2][2],
                                                                 f32x4 (&negm)[2], bool first, int kbase_key, int L,
                                                                 int g) {
  constexpr int CBLK = Bf16Tile<D>::CBLK;
  constexpr float REF_SLACK = 8.0f;
  if constexpr (MASKED) {
    const int kb0 = kbase_key + 4 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kb0 + 16 * kb + i >= L) s[kb][0][i] = s[kb][1][i] = -INFINITY;
  }
  // P with the current reference: the score accumulators started from -m
  // and the queries carry the scale, so they hold s c - m. Only on a tile
  // where the reference moves is P formed again, shifted by the move.
  auto make_p = [&](float d0, float d1, auto shift) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float d = qb ? d1 : d0;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 x = s[2 * jj + h][qb];
          if constexpr (decltype(shift)::value) x -= d;
          pk[jj][qb][2 * h] = pack_bf16x2(__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]));
          pk[jj][qb][2 * h + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2]), __builtin_amdgcn_exp2f(x[3]));
        }
      }
    }
  };
  make_p(0.f, 0.f, std::false_type{});
  // Whether the reference moves: it only does when a tile exceeds it by more
  // than REF_SLACK (and on the first tile), so p <= 2^REF_SLACK and the
  // accumulator is rescaled only on those tiles; numerator and denominator
  // share m. The common case needs only this lane's own 32 scores (any one
  // above REF_SLACK); the row maxima over the four lanes of each query are
  // formed only when some score of the wave is above it.
  float mx = __builtin_elementwise_maximum(s[0][0][0], s[0][1][0]);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[kb][0][i]), s[kb][1][i]);
  const bool any_grow = __any(first || mx > REF_SLACK);
  float alpha[2] = {1.f, 1.f};
  if (any_grow) {
    float d[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mq = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mq = __builtin_elementwise_maximum(mq, s[kb][qb][i]);
      const float mt = quad_max(mq);
      const bool grow = first || mt > REF_SLACK;
      d[qb] = grow ? mt : 0.f;
      alpha[qb] = first ? 0.f : __builtin_amdgcn_exp2f(-d[qb]);  // accumulator and sums are zero on the first tile
      m[qb] += d[qb];
      negm[qb] = f32x4{-m[qb], -m[qb], -m[qb], -m[qb]};
    }
    make_p(d[0], d[1], std::true_type{});
  }
  // The rare accumulator rescale comes last: the accumulator is not read in
  // this phase, and with the conditional update ahead of the exponentials the
  // register allocator moved all 64 accumulator registers on every tile
  // (32 v_mov_b64 per tile and wave) to merge the two paths.
  if (any_grow) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) acc[cb][qb] *= alpha[qb];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) lsv[qb] *= alpha[qb];
  }
}

template <int D, bool R3>
__global__ void __launch_bounds__(ATTN_THREADS, 2) attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int CHUNKS = Bf16Tile<D>::CHUNKS;
  constexpr int KSTEPS = Bf16Tile<D>::KSTEPS;
  constexpr int CBLK = Bf16Tile<D>::CBLK;

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
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int64_t head_row0 = int64_t(h) * a.rows + pb;  // first padded row of this (sample, head)

  // Rotated query rows of this lane as the B operand of S^T = K~ Q~^T: for
  // query block qb the lane holds query 16 qb + l16 of the wave, channels
  // 32 ks + 8 g .. +7 for every k-step ks. The rows are read from the caller's
  // q, rotated and multiplied by scale * log2(e) here (once per workgroup,
  // rounded to bf16 once); rows past the sample's end read its last token and
  // are never stored.
  bf16x8 qreg[2][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int32_t u = min(qs + 32 * wave + 16 * qb + l16, L - 1);
    int32_t row, col, frame = 0;
    if constexpr (R3) token_position3(u, a.text_len[seg], a.grid_hw[2 * seg], a.grid_hw[2 * seg + 1], row, col, frame);
    else token_position(u, a.text_len[seg], a.grid_hw[2 * seg + 1], row, col);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + int64_t(cb + u) * a.q_st + int64_t(h) * a.q_sh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const Chunk<uint16_t> raw = *reinterpret_cast<const Chunk<uint16_t>*>(qrow + 32 * ks);
      if constexpr (R3)
        qreg[qb][ks] =
            __builtin_bit_cast(bf16x8, rotate_chunk3<uint16_t, D, true>(raw, 32 * ks + 8 * g, row, col, frame, a.r3,
                                                                        a.c_log2));
      else
        qreg[qb][ks] =
            __builtin_bit_cast(bf16x8, rotate_chunk<uint16_t, D, true>(raw, 32 * ks + 8 * g, row, col, a.cs, a.c_log2));
    }
  }
  // The tile copies share the in-order vector-memory counter with these
  // loads: finish Q first so later waits only cover tile copies.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);

  // Three K~ and three V~^T tile buffers (chunk-major, verbatim copies).
  __shared__ u32x4 kA[CHUNKS], kB[CHUNKS], kC[CHUNKS], vA[CHUNKS], vB[CHUNKS], vC[CHUNKS];
  // Key tiles [kt0, kt1) of the sample; the sample's last tile carries the key mask.
  const u32x4* kg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.kw) + head_row0 * D) + kt0 * CHUNKS;
  const u32x4* vg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.vw) + head_row0 * D) + kt0 * CHUNKS;
  const int nkt = kt1 - kt0;
  const int key0 = KTILE * kt0;
  const bool mask_last = kt1 == nkt_all;

  float m[2] = {0.f, 0.f};              // reference row max (log2 units) of both queries
  f32x4 negm[2] = {f32x4{}, f32x4{}};   // -m, the score accumulators' initial value
  f32x4 lsv[2] = {f32x4{}, f32x4{}};    // row sums (every entry), accumulated by MFMAs against ones
  f32x4 acc[CBLK][2];
#pragma unroll
  for (int b = 0; b < CBLK; ++b) acc[b][0] = acc[b][1] = f32x4{};

  // Two groups of waves, 0-3 and 4-7 (waves w and w + 4 share a SIMD), run the
  // same program, for every tile j an MFMA phase (P.V of tile j-1, scores of
  // tile j) and then a VALU phase (softmax of tile j), with a barrier after
  // each phase and group 1 one barrier behind group 0: between two barriers
  // one wave of every SIMD issues MFMAs while the other runs its softmax.
  // K~(j) sits in kbuf[j % 3], V~^T(j) in vbuf[j % 3]. At the start of its VALU
  // phase of tile j every wave issues its share of the copies of K~(j+2) and
  // V~^T(j+1) (past the sample's last tile: the last tile again, into a free
  // buffer, never read), and at the end of its next MFMA phase it waits for
  // them (vmcnt(0)), so the MFMA phase carries no copy instructions. Counted
  // in phases of the two groups together (group 0's MFMA phase of tile j is
  // phase 2j, group 1's is 2j+1), a buffer is refilled only after both
  // groups' last read of it (K~(j-1) is last read in phase 2j-1, refilled from
  // phase 2j+1; V~^T(j-2) likewise), and every wave's share of K~(j+2) and
  // V~^T(j+1) has landed by the end of phase 2j+3, before the first read of
  // those tiles in phase 2j+4.
  const int grp = wave >> 2;
  f32x4 s[4][2];
  u32x4 pk[2][2];
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are complete
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_copies = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's tile copies have landed
    __builtin_amdgcn_sched_barrier(0);
  };
  const int last = nkt - 1;
  auto copy_k = [=](int t, u32x4* dst) __attribute__((always_inline)) {
    tile_to_lds<CHUNKS>(kg + min(t, last) * CHUNKS, dst, wave, lane);
  };
  auto copy_v = [=](int t, u32x4* dst) __attribute__((always_inline)) {
    tile_to_lds<CHUNKS>(vg + min(t, last) * CHUNKS, dst, wave, lane);
  };
  // Tile jt with K~(jt) in kc and V~^T(jt-1) in vp; copies of K~(jt+2) into kn
  // and V~^T(jt+1) into vn. The buffers are named statically (loop unrolled by
  // three) so that the compiler can tell the copies' targets from the tiles read.
  auto key_tile = [&](int jt, auto pv, u32x4* kc, u32x4* vp, u32x4* kn, u32x4* vn) __attribute__((always_inline)) {
    // The MFMA phase runs at raised wave priority, so that the SIMD issues its
    // MFMAs and operand reads ahead of the partner wave's softmax.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (decltype(pv)::value) mfma_phase<D, true, true>(kc, vp, qreg, acc, s, pk, lsv, negm, g, l16);
    else mfma_phase<D, false, true>(kc, vp, qreg, acc, s, pk, lsv, negm, g, l16);
    wait_copies();
    __builtin_amdgcn_s_setprio(0);
    bar();
    copy_k(jt + 2, kn);
    copy_v(jt + 1, vn);
    if (mask_last && jt == last) valu_phase<D, true>(s, acc, m, lsv, pk, negm, jt == 0, key0 + KTILE * jt, L, g);
    else valu_phase<D, false>(s, acc, m, lsv, pk, negm, jt == 0, key0 + KTILE * jt, L, g);
    bar();
  };
  using Yes = std::true_type;
  using No = std::false_type;
  copy_k(0, kA);
  copy_k(1, kB);
  copy_v(0, vA);
  wait_tile_and_sync();
  if (grp == 1) bar();
  // j % 3 == 0: K~ kA, V~^T(j-1) vC, copies into kC, vB
  // j % 3 == 1: K~ kB, V~^T(j-1) vA, copies into kA, vC
  // j % 3 == 2: K~ kC, V~^T(j-1) vB, copies into kB, vA
  key_tile(0, No{}, kA, vC, kC, vB);
  int j = 1;
  if (j < nkt) key_tile(j++, Yes{}, kB, vA, kA, vC);
  if (j < nkt) key_tile(j++, Yes{}, kC, vB, kB, vA);
  for (; j + 3 <= nkt; j += 3) {
    key_tile(j, Yes{}, kA, vC, kC, vB);
    key_tile(j + 1, Yes{}, kB, vA, kA, vC);
    key_tile(j + 2, Yes{}, kC, vB, kB, vA);
  }
  if (j < nkt) key_tile(j++, Yes{}, kA, vC, kC, vB);
  if (j < nkt) key_tile(j++, Yes{}, kB, vA, kA, vC);
  // P.V of the last tile, V~^T(last) in vbuf[last % 3].
  switch (last % 3) {
    case 0: mfma_phase<D, true, false>(kA, vA, qreg, acc, s, pk, lsv, negm, g, l16); break;
    case 1: mfma_phase<D, true, false>(kA, vB, qreg, acc, s, pk, lsv, negm, g, l16); break;
    default: mfma_phase<D, true, false>(kA, vC, qreg, acc, s, pk, lsv, negm, g, l16); break;
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): no copy into LDS left in flight
  if (grp == 0) bar();

  // Epilogue: O = acc / l. acc[b][qb] holds channels 16 b + 4 g .. +3 of query
  // 16 qb + l16 of the wave.
  float lsum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) lsum[qb] = lsv[qb][0];
  if (part >= 0) {
    // Piece of a split unit: unnormalized accumulator, reference max and row
    // sum into its slot, for the merge kernel.
    float* slot = a.part + int64_t(blockIdx.x - plan.n_full) * QTILE * (D + 2);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r = 32 * wave + 16 * qb + l16;
#pragma unroll
      for (int b = 0; b < CBLK; ++b)
        *reinterpret_cast<float4*>(slot + int64_t(r) * D + 16 * b + 4 * g) =
            make_float4(acc[b][qb][0], acc[b][qb][1], acc[b][qb][2], acc[b][qb][3]);
      if (g == 0) {
        slot[QTILE * D + r] = m[qb];
        slot[QTILE * D + QTILE + r] = lsum[qb];
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv = 1.f / lsum[qb];
    const int32_t qrel = qs + 32 * wave + 16 * qb + l16;
    if (qrel >= L) continue;
    // log-sum-exp in natural-log units: p = 2^(s c - m) / lsum, so
    // ln sum_k e^(s_k * scale) = (m + log2 lsum) * ln 2.
    if (a.lse && g == 0) a.lse[int64_t(h) * a.tokens + cb + qrel] = (m[qb] + log2f(lsum[qb])) * 0.6931471805599453f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + int64_t(cb + qrel) * a.o_st + int64_t(h) * a.o_sh + 4 * g;
#pragma unroll
    for (int b = 0; b < CBLK; ++b) {
      uint2 v2;
      v2.x = pack_bf16x2(acc[b][qb][0] * inv, acc[b][qb][1] * inv);
      v2.y = pack_bf16x2(acc[b][qb][2] * inv, acc[b][qb][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * b) = v2;
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
    uint16_t* orow = static_cast<uint16_t*>(a.out) + int64_t(cb + qs + r) * a.o_st + int64_t(h) * a.o_sh + CPL * lane;
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
    float* orow = static_cast<float*>(a.out) + int64_t(cb + qrel) * a.o_st + int64_t(h) * a.o_sh + HD * hf;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < HD; ++i) orow[i] = acc[i] * inv;
  }
}

hipError_t launch_attn_fwd(char* ws, const WsLayout& l, const void* q, const int32_t* grid_hw,
                           const int32_t* text_len, const float2* cs, const Rope3* r3, void* out, float* lse,
                           int64_t tokens, int32_t heads, int32_t head_dim, bool bf16, float scale, int32_t ncu,
                           const Strides& st, hipStream_t s) {
  AttnArgs a;
  a.ws = ws;
  a.q = q;
  a.q_st = st.q_st;
  a.q_sh = st.q_sh;
  a.o_st = st.o_st;
  a.o_sh = st.o_sh;
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
