// Shared definitions of the HIP library: tile sizes, workspace layout, token
// position rule and small device helpers. Included by every .hip source and
// by the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

// Keys per K/V tile. Every sample starts on a multiple of KTILE in the padded
// workspace layout, so tiles never straddle two samples.
constexpr int KTILE = 64;
// Queries per attention workgroup (both dtypes use the same tile table): one
// wave per 32 query rows.
#ifndef MF_QTILE
#define MF_QTILE 256
#endif
constexpr int QTILE = MF_QTILE;
constexpr int ATTN_WAVES = QTILE / 32;
constexpr int ATTN_THREADS = 64 * ATTN_WAVES;
// Positions per axis covered by the cos/sin table.
constexpr int ROPE_PMAX = 512;
constexpr int MAX_SEGMENTS = 4096;

// FLAG_REPORTED marks a failed check that mf_get_device_error has already
// returned: still not FLAG_OK (no kernel uses that header), not reported again.
enum : int32_t { FLAG_OK = 0, FLAG_METADATA = 1, FLAG_POSITION = 2, FLAG_REPORTED = 4 };

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// Rows per head of the padded Q~/K~/V^T buffers: every sample padded to a
// multiple of KTILE (at most KTILE-1 extra rows each) plus one QTILE-KTILE
// slack so the last query tile of the last sample stays inside the buffer.
__host__ __device__ inline int64_t padded_rows(int64_t tokens, int32_t n_seg) {
  return round_up(tokens + int64_t(n_seg) * (KTILE - 1), KTILE) + (QTILE - KTILE);
}

__host__ __device__ inline int64_t max_tiles(int64_t tokens, int32_t n_seg) {
  return ceil_div(tokens, QTILE) + n_seg;
}

// Split of the last partial round of (query tile, head) units over key ranges.
// With U units on ncu CUs (one workgroup per CU), the last U mod ncu units
// would run as a partly filled round as long as a whole unit. Cut into s key
// ranges (2 to 4), they take ceil(s * tail / ncu) / s of that time, plus a
// fixed cost per piece (its query load, first tile and partial write) and a
// merge kernel that combines the partial results; on a 1024x1024 batch that
// overhead measured about 60 us, some 35 key tiles of work, and erased the
// saving. So the tail is split only when that saves at least
// SPLIT_MIN_SAVED key tiles of its shortest unit (nkt_short key tiles; units
// are dispatched longest first, so the last unit is the shortest).
// Units are numbered in dispatch order: [0, n_full) whole, then n_tail units
// of `parts` pieces each. Every kernel derives the same plan from
// (U, ncu, nkt_short), so nothing is stored.
constexpr int PART_SLOTS = 512;      // partial-result slots in the workspace (pieces per call)
#ifndef MF_SPLIT_MIN_SAVED
#define MF_SPLIT_MIN_SAVED 96
#endif
constexpr int SPLIT_MIN_SAVED = MF_SPLIT_MIN_SAVED;  // key tiles a split must save on the tail's shortest unit
// A split needs a shortest unit of at least 4/3 * SPLIT_MIN_SAVED key tiles
// (4 parts in one round), i.e. a shortest sample of more than
// (4/3 * SPLIT_MIN_SAVED - 1) * KTILE tokens; the shortest sample is never
// longer than the mean, so a batch with tokens / n_seg below that cannot split
// and the host then skips the merge launch (and tells the kernel not to split).
constexpr int64_t SPLIT_MIN_MEAN_LEN = (int64_t(SPLIT_MIN_SAVED) * 4 / 3 - 1) * KTILE + 1;
__host__ __device__ inline bool split_possible(int64_t tokens, int32_t n_seg,
                                               int64_t min_saved = SPLIT_MIN_SAVED) {
  return tokens >= int64_t(n_seg) * ((min_saved * 4 / 3 - 1) * KTILE + 1);
}
// The backward's dK/dV kernel splits its last round over query ranges (64-row
// steps, each ~2.4 us of a workgroup against ~1.8 us per forward key tile,
// and a lighter merge: no rescale), so a smaller saving pays.
constexpr int SPLIT_MIN_SAVED_BWD = 24;
constexpr int BWD_KV_KEYS = 128;  // keys per dK/dV workgroup (4 groups of a dV and a dK wave)
struct SplitPlan {
  int32_t n_full, n_tail, parts;
};
__host__ __device__ inline SplitPlan split_plan(int64_t units, int32_t ncu, int64_t nkt_short,
                                               int64_t min_saved = SPLIT_MIN_SAVED) {
  SplitPlan p{int32_t(units), 0, 1};
  if (ncu <= 0 || units <= ncu) return p;
  const int64_t tail = units % ncu;
  if (tail == 0) return p;
  // Time of the tail in whole-unit times: ceil(s * tail / ncu) / s for s parts.
  int64_t best_r = 1, best_s = 1;  // rounds of pieces, parts (ratio best_r / best_s)
  for (int64_t s = 2; s <= 4 && s * tail <= PART_SLOTS; ++s) {
    const int64_t r = (s * tail + ncu - 1) / ncu;
    if (r * best_s < best_r * s) {
      best_r = r;
      best_s = s;
    }
  }
  if (best_s == 1 || nkt_short * (best_s - best_r) < min_saved * best_s) return p;
  p.n_full = int32_t(units - tail);
  p.n_tail = int32_t(tail);
  p.parts = int32_t(best_s);
  return p;
}

// XCD-aware order of the whole (query tile, head) units of the forward and
// dQ kernels. Workgroups go to the 8 XCDs round-robin by index, so with heads
// a multiple of 8 the units of one sample that land on XCD x are those of
// heads / 8 heads, every query tile of each. In tile-major order each XCD runs
// all of those heads in every round of the grid and streams their key-side
// tiles once per round; here they are reordered head-major (all tiles of one
// head, then the next), so the workgroups sharing a head's key tiles run
// together and each head is streamed about once. The permutation stays
// inside one sample's units on one XCD (equal work, longest-first order
// between samples kept), among its query tiles whose units are all whole (not
// split); results do not depend on it.
__device__ inline int xcd_unit(int unit, int heads, int tile, int qs, int32_t L, int n_full) {
  if (heads % 8 != 0) return unit;
  const int u0 = (tile - qs / QTILE) * heads;      // the sample's first unit
  // its query tiles whose units are all whole (all of them unless the split
  // last round cuts into the sample)
  const int n_s = min((L + QTILE - 1) / QTILE, (n_full - u0) / heads);
  if (unit >= u0 + n_s * heads) return unit;
  const int p = unit - u0;
  const int c = p & 7, k = p >> 3;                 // run of XCD (u0 + c) % 8, position k in it
  return u0 + (k % n_s) * heads + c + 8 * (k / n_s);
}

// Element strides of the caller's q, k, v and out: token t, head h, channel c
// of a tensor sits at t * st + h * sh + c (channels contiguous).
struct Strides {
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
};
__host__ __device__ inline Strides contiguous_strides(int32_t heads, int32_t head_dim) {
  const int64_t st = int64_t(heads) * head_dim, sh = head_dim;
  return Strides{st, sh, st, sh, st, sh, st, sh};
}

// Workspace: [header 256 B][len n][cu n+1][pcu n+1][tiles 2*max_tiles][Q~][K~][V~][partials]
// with every section 256-byte aligned. Q~, K~, V~ are [heads][rows][head_dim].
struct WsHeader {
  int32_t flag;          // FLAG_* of the last metadata check
  int32_t n_tiles;       // valid entries of the tile table
  int32_t padded_total;  // padded rows used by the samples (pcu[n])
  int32_t n_seg;
  int32_t pad[60];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

struct WsLayout {
  int64_t off_len, off_cu, off_pcu, off_tiles, off_q, off_k, off_v, off_part, total;
  int64_t rows;     // padded rows per head
  int64_t n_tiles;  // capacity of the tile table
};

// with_parts = false leaves out the partial-result slots of split units (the
// caller then never lets the attention kernel split).
__host__ __device__ inline WsLayout ws_layout(int64_t tokens, int32_t heads, int32_t head_dim,
                                              int32_t elem_bytes, int32_t n_seg, bool with_parts = true) {
  WsLayout l;
  int64_t o = 256;
  l.off_len = o;   o += round_up(int64_t(n_seg) * 4, 256);
  l.off_cu = o;    o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.off_pcu = o;   o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.n_tiles = max_tiles(tokens, n_seg);
  l.off_tiles = o; o += round_up(l.n_tiles * 8, 256);
  l.rows = padded_rows(tokens, n_seg);
  const int64_t buf = round_up(int64_t(heads) * l.rows * head_dim * elem_bytes, 256);
  l.off_q = o; o += elem_bytes == 4 ? buf : 0;  // rotated queries: fp32 path only (bf16 rotates them in the kernel)
  l.off_k = o; o += buf;
  l.off_v = o; o += buf;
  // bf16 path: PART_SLOTS partial results of split units, each QTILE rows of
  // head_dim fp32 accumulators followed by QTILE reference maxima and QTILE row sums.
  l.off_part = o; o += elem_bytes == 2 && with_parts ? int64_t(PART_SLOTS) * QTILE * (head_dim + 2) * 4 : 0;
  l.total = o;
  return l;
}

// Backward workspace: the same header, metadata and tile-table sections as
// ws_layout, then seven bf16 buffers [heads][rows][head_dim] and per-row
// statistics. Buffers (tiles of KTILE padded rows):
//   qc  Q~ chunk-major          qt  Q~^T, MFMA-order, chunk-major
//   oc  dO chunk-major          ot  dO^T, MFMA-order, chunk-major
//   kc  K~ chunk-major          kt  K~^T, MFMA-order, chunk-major
//   vc  V chunk-major
//   st  f32 [heads][rows / KTILE][2 * KTILE]: per tile, log2-domain LSE of
//       the KTILE rows (+inf on padding rows), then D = rowsum(dO * O).
struct BwdLayout {
  WsLayout m;  // metadata sections (its off_q / off_k / off_v / off_part / total are not used)
  int64_t off_qc, off_qt, off_oc, off_ot, off_kc, off_kt, off_vc, off_st, off_part, off_qpart, total;
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t tokens, int32_t heads, int32_t head_dim,
                                                int32_t n_seg) {
  BwdLayout b;
  b.m = ws_layout(tokens, heads, head_dim, 2, n_seg);
  const int64_t buf = round_up(int64_t(heads) * b.m.rows * head_dim * 2, 256);
  int64_t o = b.m.off_q;
  b.off_qc = o; o += buf;
  b.off_qt = o; o += buf;
  b.off_oc = o; o += buf;
  b.off_ot = o; o += buf;
  b.off_kc = o; o += buf;
  b.off_kt = o; o += buf;
  b.off_vc = o; o += buf;
  b.off_st = o; o += round_up(int64_t(heads) * b.m.rows * 2 * 4, 256);
  // PART_SLOTS partial dV, dK of split dK/dV units: [dV | dK][BWD_KV_KEYS keys][head_dim] fp32 each.
  b.off_part = o; o += int64_t(PART_SLOTS) * 2 * BWD_KV_KEYS * head_dim * 4;
  // PART_SLOTS partial dQ of split dQ units: [QTILE rows][head_dim] fp32 each.
  b.off_qpart = o; o += int64_t(PART_SLOTS) * QTILE * head_dim * 4;
  b.total = o;
  return b;
}

// Position of token u (counted from the start of its sample): prompt tokens
// at (0, 0), image token p = u - text_len at (p / w, p % w).
__device__ inline void token_position(int32_t u, int32_t text_len, int32_t w, int32_t& row,
                                      int32_t& col) {
  if (u < text_len) {
    row = 0;
    col = 0;
  } else {
    const int32_t p = u - text_len;
    row = p / w;
    col = p - row * w;
  }
}

// Position of token u of an editing sample (prompt, then `frames` images of
// one h x w grid): prompt tokens at (0, 0, 0), visual token p = u - text_len
// of image f = p / (h w) at (row, col) = ((p mod h w) / w, p mod w).
__device__ inline void token_position3(int32_t u, int32_t text_len, int32_t h, int32_t w, int32_t& row,
                                       int32_t& col, int32_t& frame) {
  if (u < text_len) {
    row = col = frame = 0;
  } else {
    const int32_t p = u - text_len, hw = h * w;
    frame = p / hw;
    const int32_t q = p - frame * hw;
    row = q / w;
    col = q - row * w;
  }
}

// Largest i in [0, n) with a[i] <= x, for a non-decreasing a[0..n] with a[0] <= x.
__device__ inline int32_t upper_segment(const int32_t* a, int32_t n, int64_t x) {
  int32_t lo = 0, hi = n;  // invariant a[lo] <= x < a[hi] (a[n] treated as +inf if x beyond)
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// bf16 helpers: round-to-nearest-even conversion and widening.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Swizzled position of 16-byte chunk `c` inside a tile stored as 256-byte
// lines: slot s of line L is stored at slot s ^ (L % 16). Rows read by
// 16 consecutive lanes at one logical column then hit 16 distinct bank groups.
__host__ __device__ inline int32_t swz_chunk(int32_t c) {
  const int32_t line = c >> 4;
  return (line << 4) | ((c & 15) ^ (line & 15));
}

}  // namespace mf
