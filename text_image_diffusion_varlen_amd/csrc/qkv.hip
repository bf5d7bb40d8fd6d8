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
//   qkv_rms_kernel    one wave per token: writes the token into its
//                     modality's row list and 1 / r_t.
//   qkv_gemm_kernel   per modality a GEMM over its row list: workgroup tile
//                     256 output features x 256 tokens, 8 waves of 128 x 64,
//                     v_mfma_f32_32x32x16_bf16 with D = W' X^T (lane = token),
//                     K staged 64 channels at a time in LDS by direct-to-LDS
//                     copies (the token rows are gathered through the row list
//                     by the copy itself), double-buffered; the epilogue scales
//                     by 1 / r_t and writes q, k, v rows directly.
// gamma is folded into the weight beforehand (qkv_fold_kernel:
// W' = W diag(gamma), bf16), so the normalized activations are never stored.
#include <algorithm>

#include "mf_common.h"
#include "mfma_util.h"

namespace mf {

constexpr int QKV_THREADS = 512;                  // 8 waves
constexpr int QKV_NT = 256;                       // output features per workgroup
constexpr int QKV_TT = 256;                       // tokens per workgroup
constexpr int QKV_KS = 64;                        // hidden channels per LDS stage
constexpr int QKV_CH = QKV_NT * QKV_KS / 8;       // 16-byte chunks per operand tile
static_assert(QKV_TT == QKV_NT, "A and B tiles share one copy pattern");
constexpr int ROUTE_THREADS = 1024;

struct QkvHeader {
  int32_t flag;   // FLAG_OK or FLAG_METADATA
  int32_t n_txt;  // prompt tokens of the batch
  int32_t n_img;  // visual tokens of the batch
  int32_t pad[61];
};
static_assert(sizeof(QkvHeader) == 256, "one 256-byte block");

// Workspace: [header][tp n+1][vp n+1][idx_txt T][idx_img T][inv_r T], 256-byte aligned sections.
struct QkvLayout {
  int64_t off_tp, off_vp, off_txt, off_img, off_inv, total;
};
__host__ __device__ inline QkvLayout qkv_layout(int64_t tokens, int32_t n_seg) {
  QkvLayout l;
  int64_t o = 256;
  l.off_tp = o;  o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.off_vp = o;  o += round_up(int64_t(n_seg + 1) * 4, 256);
  l.off_txt = o; o += round_up(tokens * 4, 256);
  l.off_img = o; o += round_up(tokens * 4, 256);
  l.off_inv = o; o += round_up(tokens * 4, 256);
  l.total = o;
  return l;
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

// One wave per token: its place in its modality's row list and 1 / r_t.
__global__ void __launch_bounds__(256)
qkv_rms_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, const int32_t* __restrict__ text_len,
               int32_t n, int64_t tokens, int32_t hidden, float eps, char* __restrict__ ws, QkvLayout l) {
  const QkvHeader* hdr = reinterpret_cast<const QkvHeader*>(ws);
  if (hdr->flag != FLAG_OK) return;
  const int64_t tok = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= tokens) return;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + tok * hidden);
  float ss = 0.f;
  for (int c = lane; c < hidden / 8; c += 64) {
    const u32x4 r = row[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(r[e] << 16), b = __uint_as_float(r[e] & 0xFFFF0000u);
      ss = __builtin_fmaf(a, a, __builtin_fmaf(b, b, ss));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) {
    const int32_t i = upper_segment(cu, n, tok);
    const int32_t u = int32_t(tok - cu[i]);
    const int32_t* tp = reinterpret_cast<const int32_t*>(ws + l.off_tp);
    const int32_t* vp = reinterpret_cast<const int32_t*>(ws + l.off_vp);
    if (u < text_len[i]) reinterpret_cast<int32_t*>(ws + l.off_txt)[tp[i] + u] = int32_t(tok);
    else reinterpret_cast<int32_t*>(ws + l.off_img)[vp[i] + u - text_len[i]] = int32_t(tok);
    reinterpret_cast<float*>(ws + l.off_inv)[tok] = 1.0f / sqrtf(ss / float(hidden) + eps);
  }
}

// W'_m[n][c] = bf16(gamma_m[c] * W_m[n][c]) for both modalities.
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
  const u32x4 r = *reinterpret_cast<const u32x4*>(src);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __uint_as_float(r[e] << 16) * g[2 * e];
    const float b = __uint_as_float(r[e] & 0xFFFF0000u) * g[2 * e + 1];
    o[e] = pack_bf16x2(a, b);
  }
  *reinterpret_cast<u32x4*>(out + e0) = o;
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
  int32_t hd;          // heads * head_dim
  int32_t n_tiles;     // 3 hd / QKV_NT
};

__global__ void __launch_bounds__(QKV_THREADS, 2) qkv_gemm_kernel(QkvGemmArgs a) {
  const QkvHeader* hdr = reinterpret_cast<const QkvHeader*>(a.ws);
  if (hdr->flag != FLAG_OK) return;
  const int nt = int(blockIdx.x % unsigned(a.n_tiles));
  int tt = int(blockIdx.x / unsigned(a.n_tiles));
  const int32_t n_txt = hdr->n_txt, n_img = hdr->n_img;
  const int txt_tiles = (n_txt + QKV_TT - 1) / QKV_TT;
  int m = 0;
  int32_t count = n_txt;
  if (tt >= txt_tiles) {
    tt -= txt_tiles;
    m = 1;
    count = n_img;
    if (tt * QKV_TT >= n_img) return;
  }
  const int32_t* rows = reinterpret_cast<const int32_t*>(a.ws + (m ? a.l.off_img : a.l.off_txt));
  const int32_t row0 = tt * QKV_TT;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int wn = wave & 1, wt = wave >> 1;  // wave tile: 128 features x 64 tokens

  // Copy pattern (both operands): wave w moves chunk w (channels 8w .. 8w+7 of
  // the stage) of all 256 rows, one 64-row block per instruction; LDS is
  // chunk-major (chunk c of row r at c * 256 + r).
  const int64_t K = a.hidden;
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * i + lane;
    wsrc[i] = a.w + (int64_t(m) * 3 * a.hd + int64_t(nt) * QKV_NT + r) * K + 8 * wave;
    const int32_t tok = rows[min(row0 + r, count - 1)];  // rows past the list repeat its last token (not stored)
    xsrc[i] = a.x + int64_t(tok) * K + 8 * wave;
  }
  __shared__ u32x4 lds[2][2 * QKV_CH];  // [stage][A (features) | B (tokens)]
  auto load_stage = [&](int s, u32x4* dst) {
    const int64_t k0 = int64_t(s) * QKV_KS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(wsrc[i] + k0),
                                       (lds_ptr_t)(dst + wave * QKV_NT + 64 * i), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(xsrc[i] + k0),
                                       (lds_ptr_t)(dst + QKV_CH + wave * QKV_NT + 64 * i), 16, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb][0] = acc[nb][1] = f32x16{};
  const int stages = a.hidden / QKV_KS;
  load_stage(0, lds[0]);
  wait_vm_and_sync();
  for (int s = 0; s < stages; ++s) {
    const u32x4* cur = lds[s & 1];
    if (s + 1 < stages) load_stage(s + 1, lds[(s + 1) & 1]);
    const u32x4* al = cur + hf * QKV_NT + wn * 128 + l32;
    const u32x4* bl = cur + QKV_CH + hf * QKV_NT + wt * 64 + l32;
#pragma unroll
    for (int ks = 0; ks < QKV_KS / 16; ++ks) {
      bf16x8 bo[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) bo[tb] = as_bf16x8(bl[2 * QKV_NT * ks + 32 * tb]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 ao = as_bf16x8(al[2 * QKV_NT * ks + 32 * nb]);
        acc[nb][0] = mfma32(ao, bo[0], acc[nb][0]);
        acc[nb][1] = mfma32(ao, bo[1], acc[nb][1]);
      }
    }
    wait_vm_and_sync();
  }

  // Epilogue: lane = token, entry e of block nb = feature 32nb + 8(e/4) + 4hf + e%4.
  const float* inv = reinterpret_cast<const float*>(a.ws + a.l.off_inv);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int32_t row = row0 + wt * 64 + tb * 32 + l32;
    if (row >= count) continue;
    const int32_t tok = rows[row];
    const float sc = inv[tok];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nt * QKV_NT + wn * 128 + nb * 32 + 8 * g + 4 * hf;
        const int which = n / a.hd, rem = n - which * a.hd;
        uint16_t* dst = (which == 0 ? a.q : which == 1 ? a.k : a.v) + int64_t(tok) * a.hd + rem;
        uint2 o;
        o.x = pack_bf16x2(acc[nb][tb][4 * g] * sc, acc[nb][tb][4 * g + 1] * sc);
        o.y = pack_bf16x2(acc[nb][tb][4 * g + 2] * sc, acc[nb][tb][4 * g + 3] * sc);
        *reinterpret_cast<uint2*>(dst) = o;
      }
    }
  }
}

size_t qkv_workspace_bytes(int64_t tokens, int32_t n_seg) { return size_t(qkv_layout(tokens, n_seg).total); }

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
                      char* ws, void* q, void* k, void* v, hipStream_t s, hipEvent_t const* ev) {
  const QkvLayout l = qkv_layout(tokens, n_seg);
  hipError_t e;
  hipLaunchKernelGGL(qkv_route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, s, cu, grid_hw, text_len, frames, n_seg,
                     tokens, ws, l);
  hipLaunchKernelGGL(qkv_rms_kernel, dim3(unsigned(ceil_div(tokens, 4))), dim3(256), 0, s,
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
  a.hd = hd;
  a.n_tiles = 3 * hd / QKV_NT;
  // Token tiles of both modalities together never exceed ceil(T / 256) + 1.
  const int64_t tiles = (ceil_div(tokens, QKV_TT) + 1) * a.n_tiles;
  hipLaunchKernelGGL(qkv_gemm_kernel, dim3(unsigned(tiles)), dim3(QKV_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace mf
