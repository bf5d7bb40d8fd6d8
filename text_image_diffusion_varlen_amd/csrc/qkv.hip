// Modality-specific RMSNorm + packed QKV projection of a packed batch.
//
// Sources: Mage-Flow tech report, NR-MMDiT section (every MMDiT block has
// separate normalization and projection layers for the text and the visual
// stream; the streams meet only in the joint attention); mageflow.net
// architecture page, section 7 (fused RMSNorm, packed linear projections).
// For token t of modality m (prompt token: text, otherwise visual):
//   r_t = sqrt(mean_c x[t][c]^2 + eps),
//   [q | k | v][t][n] = sum_c x[t][c] / r_t * gamma_m[c] * W_m[n][c],
// W_m [3 H d][hidden] stored as a linear layer's weight (rows: q, then k,
// then v, each head-major), q, k, v written as [T][H][d].
//
// Three kernels:
//   qkv_route_kernel  (one workgroup) checks the metadata and counts each
//                     sample's prompt and visual tokens (prefix sums).
//   qkv_rms_kernel    per 64 rows of one modality: the rows' tokens, 1 / r_t,
//                     the row lists, and the rows copied into the tiled
//                     activation buffer X~ (text rows, then visual rows).
//   qkv_gemm_kernel   per modality a GEMM over its rows: workgroup tile 256
//                     output features x 256 tokens, 8 waves of 128 x 64,
//                     v_mfma_f32_16x16x32_bf16 with D = W' X^T (lane = token),
//                     K staged 64 channels at a time in LDS by direct-to-LDS
//                     copies, double-buffered; the epilogue scales by 1 / r_t
//                     and writes q, k, v rows directly. A last round that
//                     would fill at most half the CUs runs as 128-feature
//                     halves of its tiles (same summation order). Workgroups
//                     are mapped to tiles so that those running together on
//                     one XCD (one L2) share operand tiles.
// Both GEMM operands are stored tiled: for every 256-row x 64-channel tile,
// 2048 16-byte chunks, chunk c (channels 8c .. 8c+7) of row r at c * 256 + r.
// A stage is then one contiguous 32 KB copy per operand, and the LDS image
// gives conflict-free MFMA operand reads at immediate offsets. gamma is folded
// into the weight beforehand (qkv_fold_kernel: W' = W diag(gamma), bf16, tiled).
#include <algorithm>

#include "mf_common.h"
#include "mfma_util.h"

namespace mf {

constexpr int QKV_THREADS = 512;                  // 8 waves
constexpr int QKV_NT = 256;                       // output features per workgroup
constexpr int QKV_TT = 256;                       // tokens per workgroup
constexpr int QKV_KS = 64;                        // hidden channels per LDS stage
constexpr int QKV_CH = QKV_NT * QKV_KS / 8;       // 16-byte chunks per operand tile
constexpr int QKV_GROUP_TT = 4;                   // token tiles per group of the XCD-aware order
static_assert(QKV_TT == QKV_NT, "A and B tiles share one copy pattern");
constexpr int ROUTE_THREADS = 1024;

struct QkvHeader {
  int32_t flag;   // FLAG_OK or FLAG_METADATA
  int32_t n_txt;  // prompt tokens of the batch
  int32_t n_img;  // visual tokens of the batch
  int32_t pad[61];
};
static_assert(sizeof(QkvHeader) == 256, "one 256-byte block");

// Workspace: [header][tp n+1][vp n+1][idx_txt T][idx_img T][ssq T x G][X~], 256-byte
// aligned sections. ssq holds each token's sum of squares in G partial sums
// (one per group of RMS_STAGES channel stages). X~ holds the text rows from
// tile 0 and the visual rows from the first tile after them: at most
// ceil(T / 256) + 1 tiles of 256 x hidden.
constexpr int RMS_STAGES = 8;  // 64-channel stages per statistics workgroup
__host__ __device__ inline int32_t rms_groups(int32_t hidden) {
  return int32_t(ceil_div(hidden / QKV_KS, RMS_STAGES));
}
struct QkvLayout {
  int64_t off_tp, off_vp, off_txt, off_img, off_inv, off_x, total;
};
__host__ __device__ inline QkvLayout qkv_layout(int64_t tokens, int32_t n_seg, int32_t hidden) {
  QkvLayout l;
  int64_t o = 256;
  l.off_tp = o;  o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.off_vp = o;  o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.off_txt = o; o += round_up(tokens * 4, 256);
  l.off_img = o; o += round_up(tokens * 4, 256);
  l.off_inv = o; o += round_up(tokens * rms_groups(hidden) * 4, 256);
  l.off_x = o;   o += (ceil_div(tokens, QKV_TT) + 1) * QKV_TT * int64_t(hidden) * 2;
  l.total = o;
  return l;
}

// Chunk index of (row, 8-channel chunk cg) in a tiled operand with `stages`
// 64-channel stages per 256-row tile.
__host__ __device__ inline int64_t tiled_chunk(int64_t row, int64_t cg, int64_t stages) {
  return ((row / QKV_TT) * stages + cg / 8) * QKV_CH + (cg % 8) * QKV_TT + row % QKV_TT;
}

// Prompt / visual token counts of every sample, their exclusive prefix sums
// (tp, vp), and the check of cu_seqlens against them.
__global__ void __launch_bounds__(ROUTE_THREADS)
qkv_route_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ grid_hw,
                 const int32_t* __restrict__ text_len, const int32_t* __restrict__ frames, int32_t n,
                 int64_t tokens, char* __restrict__ ws, QkvLayout l) {
  __shared__ int64_t sc_t[ROUTE_THREADS], sc_v[ROUTE_THREADS];
  __shared__ int32_t bad;
  QkvHeader* hdr = reinterpret_cast<QkvHeader*>(ws);
  int32_t* tp = reinterpret_cast<int32_t*>(ws + l.off_tp);
  int32_t* vp = reinterpret_cast<int32_t*>(ws + l.off_vp);
  const int t = threadIdx.x;
  if (t == 0) bad = 0;
  __syncthreads();
  const int per = (n + ROUTE_THREADS - 1) / ROUTE_THREADS;
  const int b0 = min(t * per, n), b1 = min(b0 + per, n);
  int64_t lt = 0, lv = 0;
  for (int i = b0; i < b1; ++i) {
    const int32_t h = grid_hw[2 * i], w = grid_hw[2 * i + 1], tl = text_len[i], f = frames ? frames[i] : 1;
    const bool ok = h >= 1 && w >= 1 && h <= ROPE_PMAX && w <= ROPE_PMAX && tl >= 0 && tl <= (1 << 30) && f >= 1 &&
                    f <= ROPE_PMAX && int64_t(cu[i + 1]) - cu[i] == int64_t(tl) + int64_t(f) * h * w;
    if (!ok) bad = 1;
    lt += ok ? tl : 0;
    lv += ok ? int64_t(f) * h * w : 0;
  }
  sc_t[t] = lt;
  sc_v[t] = lv;
  __syncthreads();
  for (int off = 1; off < ROUTE_THREADS; off <<= 1) {
    const int64_t yt = t >= off ? sc_t[t - off] : 0, yv = t >= off ? sc_v[t - off] : 0;
    __syncthreads();
    sc_t[t] += yt;
    sc_v[t] += yv;
    __syncthreads();
  }
  int64_t rt = sc_t[t] - lt, rv = sc_v[t] - lv;
  for (int i = b0; i < b1; ++i) {
    tp[i] = int32_t(rt);
    vp[i] = int32_t(rv);
    const int32_t h = grid_hw[2 * i], w = grid_hw[2 * i + 1], f = frames ? frames[i] : 1;
    rt += text_len[i];
    rv += int64_t(f) * h * w;
  }
  if (t == 0) {
    const int64_t nt = sc_t[ROUTE_THREADS - 1], nv = sc_v[ROUTE_THREADS - 1];
    const bool ok = !bad && cu[0] == 0 && int64_t(cu[n]) == tokens && nt + nv == tokens;
    tp[n] = int32_t(nt);
    vp[n] = int32_t(nv);
    hdr->flag = ok ? FLAG_OK : FLAG_METADATA;
    hdr->n_txt = ok ? int32_t(nt) : 0;
    hdr->n_img = ok ? int32_t(nv) : 0;
  }
}

// One workgroup per (64 consecutive rows of one modality (text rows, then
// visual rows), group of RMS_STAGES channel stages): finds each row's token,
// copies its part of the rows into X~ one 64-channel stage at a time through
// LDS (row-contiguous reads, tile-contiguous writes), and writes the rows'
// partial sums of squares; the first group also writes the row lists. The
// partial sums are added in group order by the GEMM epilogue (deterministic).
constexpr int RMS_ROWS = 64;
__global__ void __launch_bounds__(256)
qkv_rms_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, const int32_t* __restrict__ text_len,
               int32_t n, int64_t tokens, int32_t hidden, float eps, char* __restrict__ ws, QkvLayout l) {
  const QkvHeader* hdr = reinterpret_cast<const QkvHeader*>(ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t n_txt = hdr->n_txt, n_img = hdr->n_img;
  const int txt_blocks = (n_txt + RMS_ROWS - 1) / RMS_ROWS;
  const int32_t groups = rms_groups(hidden);
  const int grp = int(blockIdx.x % unsigned(groups));
  int blk = int(blockIdx.x / unsigned(groups));
  const bool is_text = blk < txt_blocks;
  if (!is_text) {
    blk -= txt_blocks;
    if (blk * RMS_ROWS >= n_img) return;
  }
  const int32_t count = is_text ? n_txt : n_img;
  const int32_t* pre = reinterpret_cast<const int32_t*>(ws + (is_text ? l.off_tp : l.off_vp));
  const int32_t r0 = blk * RMS_ROWS;
  const int64_t t0 = is_text ? r0 : round_up(n_txt, QKV_TT) + r0;  // X~ row of this block's first row
  const int t = threadIdx.x;
  __shared__ int32_t tok_of[RMS_ROWS];
  __shared__ float ssq[RMS_ROWS];
  __shared__ u32x4 stage[8 * RMS_ROWS];  // chunk c of row r at c * 64 + r
  if (t < RMS_ROWS) {
    const int32_t rank = min(r0 + t, count - 1);
    const int32_t i = upper_segment(pre, n, rank);  // pre[] is non-decreasing, pre[0] = 0
    tok_of[t] = cu[i] + (is_text ? 0 : text_len[i]) + (rank - pre[i]);
  }
  __syncthreads();
  const int64_t stages = hidden / QKV_KS;
  u32x4* xt = reinterpret_cast<u32x4*>(ws + l.off_x);
  float ss[2] = {0.f, 0.f};
  const int64_t s_end = min(stages, int64_t(grp + 1) * RMS_STAGES);
  for (int64_t s = int64_t(grp) * RMS_STAGES; s < s_end; ++s) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 512 chunks: 8 per row, 8 consecutive threads per row
      const int q = t + 256 * j, r = q >> 3, c = q & 7;
      const u32x4 v = reinterpret_cast<const u32x4*>(x + int64_t(tok_of[r]) * hidden)[8 * s + c];
      stage[c * RMS_ROWS + r] = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __uint_as_float(v[e] << 16), b = __uint_as_float(v[e] & 0xFFFF0000u);
        ss[j] = __builtin_fmaf(a, a, __builtin_fmaf(b, b, ss[j]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = t + 256 * j, c = q / RMS_ROWS, r = q % RMS_ROWS;
      const int64_t row = t0 + r;
      xt[((row / QKV_TT) * stages + s) * QKV_CH + c * QKV_TT + row % QKV_TT] = stage[c * RMS_ROWS + r];
    }
    __syncthreads();
  }
  // Rows t/8 and t/8 + 32: sum over the 8 threads of each row.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int o = 4; o >= 1; o >>= 1) ss[j] += __shfl_xor(ss[j], o, 64);
    if ((t & 7) == 0) ssq[(t >> 3) + 32 * j] = ss[j];
  }
  __syncthreads();
  if (t < RMS_ROWS && r0 + t < count) {
    const int32_t tok = tok_of[t];
    if (grp == 0) reinterpret_cast<int32_t*>(ws + (is_text ? l.off_txt : l.off_img))[r0 + t] = tok;
    reinterpret_cast<float*>(ws + l.off_inv)[int64_t(tok) * groups + grp] = ssq[t];
  }
}

// W'_m[n][c] = bf16(gamma_m[c] * W_m[n][c]) for both modalities, stored tiled
// (rows n of modality m at row m * out_features + n).
__global__ void __launch_bounds__(256)
qkv_fold_kernel(const uint16_t* __restrict__ w_txt, const uint16_t* __restrict__ w_img,
                const float* __restrict__ g_txt, const float* __restrict__ g_img, int64_t per_modality,
                int32_t hidden, uint16_t* __restrict__ out) {
  const int64_t chunk = int64_t(blockIdx.x) * 256 + threadIdx.x;  // 8 elements each
  if (chunk >= 2 * per_modality / 8) return;
  const int64_t e0 = chunk * 8;
  const bool img = e0 >= per_modality;
  const int64_t local = img ? e0 - per_modality : e0;
  const uint16_t* src = (img ? w_img : w_txt) + local;
  const float* g = (img ? g_img : g_txt) + local % hidden;
  const int64_t grow = e0 / hidden, cg = (e0 % hidden) / 8;  // row of the stacked [2 * out_features] weight
  const u32x4 r = *reinterpret_cast<const u32x4*>(src);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __uint_as_float(r[e] << 16) * g[2 * e];
    const float b = __uint_as_float(r[e] & 0xFFFF0000u) * g[2 * e + 1];
    o[e] = pack_bf16x2(a, b);
  }
  reinterpret_cast<u32x4*>(out)[tiled_chunk(grow, cg, hidden / QKV_KS)] = o;
}

struct QkvGemmArgs {
  const uint16_t* x;   // [T][hidden]
  const uint16_t* w;   // [2][3HD][hidden], gamma folded
  const char* ws;
  QkvLayout l;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int32_t hidden;
  float eps;
  int32_t hd;          // heads * head_dim
  int32_t n_tiles;     // 3 hd / QKV_NT
  int32_t ncu;         // compute units for the halved last round (0: never halve)
};

// One GEMM unit (256 output features x 256 tokens of one modality) or, with
// NB = 4, one 128-feature half of it starting at feature fbase of the tile:
// every wave owns NB * 16 features x 64 tokens, on v_mfma_f32_16x16x32_bf16
// (which sustains a higher rate on this chip than the 32 x 32 form). Both
// halves copy the whole stages (the tiled layout keeps a stage contiguous) and
// read their features. Per output element the products are summed in the
// same stage and k-step order in both forms, so a half unit's outputs equal
// the whole unit's bit for bit.
template <int NB>
__device__ inline void qkv_gemm_unit(const QkvGemmArgs& a, const QkvHeader* hdr, int unit, int fbase,
                                     u32x4 (*lds)[2 * QKV_CH]) {
  const int nt = unit % a.n_tiles;
  int tt = unit / a.n_tiles;
  const int32_t n_txt = hdr->n_txt, n_img = hdr->n_img;
  const int txt_tiles = (n_txt + QKV_TT - 1) / QKV_TT;
  int m = 0;
  int32_t count = n_txt;
  if (tt >= txt_tiles) {
    tt -= txt_tiles;
    m = 1;
    count = n_img;
  }
  const int32_t* rows = reinterpret_cast<const int32_t*>(a.ws + (m ? a.l.off_img : a.l.off_txt));
  const int32_t row0 = tt * QKV_TT;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wt = wave >> 1;                     // 64-token quarter
  const int fw = fbase + (wave & 1) * NB * 16;  // this wave's first feature in the tile

  // Both operands are tiled: a stage of one operand is 2048 contiguous chunks,
  // copied verbatim (chunk c of row r lands at c * 256 + r).
  const int64_t stages_k = a.hidden / QKV_KS;
  const int64_t xtile = m ? round_up(n_txt, QKV_TT) / QKV_TT + tt : tt;  // tile row of X~
  const u32x4* wsrc = reinterpret_cast<const u32x4*>(a.w) + (int64_t(m) * a.n_tiles + nt) * stages_k * QKV_CH;
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(a.ws + a.l.off_x) + xtile * stages_k * QKV_CH;
  auto load_stage = [&](int s, u32x4* dst) {
    copy_to_lds<QKV_CH, QKV_THREADS / 64>(wsrc + int64_t(s) * QKV_CH, dst, wave, lane);
    copy_to_lds<QKV_CH, QKV_THREADS / 64>(xsrc + int64_t(s) * QKV_CH, dst + QKV_CH, wave, lane);
  };

  f32x4 acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x4{};
  const int stages = a.hidden / QKV_KS;
  load_stage(0, lds[0]);
  wait_vm_and_sync();
  for (int s = 0; s < stages; ++s) {
    const u32x4* cur = lds[s & 1];
    if (s + 1 < stages) load_stage(s + 1, lds[(s + 1) & 1]);
    // Lane (g, l16) reads chunk 4 ks + g of row l16 of every 16-row block.
    const u32x4* al = cur + g * QKV_NT + fw + l16;
    const u32x4* bl = cur + QKV_CH + g * QKV_TT + wt * 64 + l16;
#pragma unroll
    for (int ks = 0; ks < QKV_KS / 32; ++ks) {
      bf16x8 bo[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) bo[tb] = as_bf16x8(bl[4 * QKV_TT * ks + 16 * tb]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 ao = as_bf16x8(al[4 * QKV_NT * ks + 16 * nb]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = mfma16(ao, bo[tb], acc[nb][tb]);
      }
    }
    wait_vm_and_sync();
  }

  // Epilogue: lane (g, l16) holds features fw + 16 nb + 4 g .. +3 of token
  // wt * 64 + 16 tb + l16 in acc[nb][tb].
  const float* ssq = reinterpret_cast<const float*>(a.ws + a.l.off_inv);
  const int32_t groups = rms_groups(a.hidden);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int32_t row = row0 + wt * 64 + tb * 16 + l16;
    if (row >= count) continue;
    const int32_t tok = rows[row];
    float ss = 0.f;
    for (int gg = 0; gg < groups; ++gg) ss += ssq[int64_t(tok) * groups + gg];
    const float sc = 1.0f / sqrtf(ss / float(a.hidden) + a.eps);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = nt * QKV_NT + fw + nb * 16 + 4 * g;
      const int which = n / a.hd, rem = n - which * a.hd;
      uint16_t* dst = (which == 0 ? a.q : which == 1 ? a.k : a.v) + int64_t(tok) * a.hd + rem;
      uint2 o;
      o.x = pack_bf16x2(acc[nb][tb][0] * sc, acc[nb][tb][1] * sc);
      o.y = pack_bf16x2(acc[nb][tb][2] * sc, acc[nb][tb][3] * sc);
      *reinterpret_cast<uint2*>(dst) = o;
    }
  }
}

// XCD-aware order of the units. Workgroups are dispatched to the 8 XCDs
// round-robin by index, and each XCD has its own L2, so the ~32 workgroups
// one XCD runs together should share operand tiles. Positions are laid out
// in groups of QKV_GROUP_TT token tiles, feature tile major inside a group,
// so 32 consecutive positions cover 8 feature tiles x 4 token tiles (12
// distinct 32 KB operand tiles per stage instead of ~17 in index order), and
// inside every whole group of 256 workgroups the 32 of one XCD take 32
// consecutive positions. Both maps are bijections, so every unit is computed
// exactly once and the outputs do not depend on the order.
__device__ inline int unit_at(int pos, int n_tiles, int token_tiles) {
  const int gsz = QKV_GROUP_TT * n_tiles;
  const int g = pos / gsz, r = pos % gsz;
  const int gs = min(QKV_GROUP_TT, token_tiles - g * QKV_GROUP_TT);  // token tiles in this group
  return (g * QKV_GROUP_TT + r % gs) * n_tiles + r / gs;
}
__device__ inline int xcd_position(int b, int n_whole) {
  const int g0 = b & ~255;
  if (g0 + 256 > n_whole) return b;
  return g0 + 32 * (b & 7) + ((b & 255) >> 3);
}

// Units = feature tiles x (text + visual token tiles), one workgroup per unit
// (one per CU: 128 KB of LDS). When the last round of units would occupy at
// most half of the a.ncu compute units, its units run as two 128-feature
// halves each, so that round takes about half as long. a.ncu = 0: never.
__global__ void __launch_bounds__(QKV_THREADS, 2) qkv_gemm_kernel(QkvGemmArgs a) {
  const QkvHeader* hdr = reinterpret_cast<const QkvHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const int32_t units = ((hdr->n_txt + QKV_TT - 1) / QKV_TT + (hdr->n_img + QKV_TT - 1) / QKV_TT) * a.n_tiles;
  const int32_t tail = a.ncu > 0 ? units % a.ncu : 0;
  const bool halve = tail > 0 && 2 * tail <= a.ncu;
  const int32_t n_full = halve ? units - tail : units;
  __shared__ u32x4 lds[2][2 * QKV_CH];  // [stage][A (features) | B (tokens)]
  const int b = int(blockIdx.x);
  const int token_tiles = units / a.n_tiles;
  if (b < n_full) {
    qkv_gemm_unit<8>(a, hdr, unit_at(xcd_position(b, n_full), a.n_tiles, token_tiles), 0, lds);
  } else if (halve && b < n_full + 2 * tail) {
    const int piece = b - n_full;
    qkv_gemm_unit<4>(a, hdr, unit_at(n_full + piece / 2, a.n_tiles, token_tiles), (piece % 2) * (QKV_NT / 2), lds);
  }
}

size_t qkv_workspace_bytes(int64_t tokens, int32_t n_seg, int32_t hidden) {
  return size_t(qkv_layout(tokens, n_seg, hidden).total);
}

hipError_t launch_qkv_fold(const void* w_txt, const void* w_img, const float* g_txt, const float* g_img,
                           int32_t hidden, int32_t out_features, void* out, hipStream_t s) {
  const int64_t per = int64_t(out_features) * hidden;
  hipLaunchKernelGGL(qkv_fold_kernel, dim3(unsigned(ceil_div(2 * per / 8, 256))), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_txt), static_cast<const uint16_t*>(w_img), g_txt, g_img, per,
                     hidden, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_qkv(const void* x, const void* w, const int32_t* cu, const int32_t* grid_hw, const int32_t* text_len,
                      const int32_t* frames, int32_t n_seg, int64_t tokens, int32_t hidden, int32_t hd, float eps,
                      char* ws, void* q, void* k, void* v, int32_t ncu, hipStream_t s, hipEvent_t const* ev) {
  const QkvLayout l = qkv_layout(tokens, n_seg, hidden);
  hipError_t e;
  hipLaunchKernelGGL(qkv_route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, s, cu, grid_hw, text_len, frames, n_seg,
                     tokens, ws, l);
  // Row blocks of both modalities together never exceed ceil(T / 64) + 1.
  hipLaunchKernelGGL(qkv_rms_kernel, dim3(unsigned((ceil_div(tokens, RMS_ROWS) + 1) * rms_groups(hidden))), dim3(256),
                     0, s,
                     static_cast<const uint16_t*>(x), cu, text_len, n_seg, tokens, hidden, eps, ws, l);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  QkvGemmArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.ws = ws;
  a.l = l;
  a.q = static_cast<uint16_t*>(q);
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.hidden = hidden;
  a.eps = eps;
  a.hd = hd;
  a.n_tiles = 3 * hd / QKV_NT;
  a.ncu = ncu;
  // Text tiles + visual tiles is ceil(T / 256) or ceil(T / 256) + 1 (the split
  // of T between the modalities is known on the device only); a halved last
  // round adds its tail count of workgroups.
  const int64_t lo = ceil_div(tokens, QKV_TT) * a.n_tiles, hi = lo + a.n_tiles;
  auto extra = [&](int64_t units) {
    const int64_t tail = ncu > 0 ? units % ncu : 0;
    return tail > 0 && 2 * tail <= ncu ? tail : 0;
  };
  hipLaunchKernelGGL(qkv_gemm_kernel, dim3(unsigned(hi + std::max(extra(lo), extra(hi)))), dim3(QKV_THREADS), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace mf
