// Packing metadata on the device.
//
// Samples are packed back to back and attention is kept inside each sample
// by per-sample cumulative offsets (Mage-Flow tech report, NR-MMDiT section,
// native-resolution packing paragraph). Sample i is its prompt followed by
// its flattened h_i x w_i latent grid, so L_i = text_len_i + h_i * w_i; an
// editing sample (same section, editing paragraph) carries f_i images of one
// grid after its prompt, L_i = text_len_i + f_i * h_i * w_i (f_i = 1 when no
// frame counts are given).
//
// meta_kernel (one workgroup) validates the caller's offsets and builds what
// the prologue and the attention kernel need:
//   len[i]   = L_i
//   cu[i]    = caller's offsets (checked against the prefix sums of L_i)
//   pcu[i]   = offsets of the padded layout, each sample rounded up to KTILE
//   tiles[]  = (sample, first query row) of every QTILE-row query tile,
//              samples in order of decreasing L_i (longest processing time
//              first), so the heaviest workgroups are dispatched first.
// positions_kernel writes the per-token (row, col) (or (row, col, frame)) and
// sample id.
#include "mf_common.h"
#include "meta_small.h"

namespace mf {

constexpr int META_THREADS = 1024;
constexpr int META_PER_THREAD = MAX_SEGMENTS / META_THREADS;  // 4

// Inclusive scan of per-thread totals across the workgroup (Hillis-Steele in LDS).
__device__ inline int64_t block_inclusive_scan(int64_t x, int64_t* buf) {
  const int t = threadIdx.x;
  buf[t] = x;
  __syncthreads();
  for (int off = 1; off < META_THREADS; off <<= 1) {
    const int64_t y = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += y;
    __syncthreads();
  }
  const int64_t r = buf[t];
  __syncthreads();
  return r;
}

// Exclusive prefix sums of this thread's META_PER_THREAD values (entries
// t*META_PER_THREAD + e, zero past the end) across the workgroup. Writes the
// exclusive sums to excl[] and returns the grand total (same on every thread).
__device__ inline int64_t block_prefix(const int64_t (&mine)[META_PER_THREAD],
                                       int64_t (&excl)[META_PER_THREAD], int64_t* buf,
                                       int64_t* total_slot) {
  int64_t local = 0;
  for (int e = 0; e < META_PER_THREAD; ++e) local += mine[e];
  const int64_t incl = block_inclusive_scan(local, buf);
  int64_t run = incl - local;
  for (int e = 0; e < META_PER_THREAD; ++e) {
    excl[e] = run;
    run += mine[e];
  }
  if (threadIdx.x == META_THREADS - 1) *total_slot = incl;
  __syncthreads();
  const int64_t total = *total_slot;
  __syncthreads();
  return total;
}

struct MetaShared {
  int32_t len[MAX_SEGMENTS];
  int32_t pre[MAX_SEGMENTS + 1];
  int32_t order[MAX_SEGMENTS];
  int64_t scan[META_THREADS];
  int64_t total;
  int32_t bad;
};

// L_i of every sample into sh.len (1 for an invalid sample) and the range checks.
__device__ inline void load_lengths(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                    int32_t n, MetaShared& sh) {
  const int t = threadIdx.x;
  if (t == 0) sh.bad = 0;
  __syncthreads();
  for (int i = t; i < n; i += META_THREADS) {
    bool ok;
    sh.len[i] = sample_length(grid_hw, text_len, frames, i, ok);
    if (!ok) atomicOr(&sh.bad, 1);
  }
  __syncthreads();
}

// Prefix sums of sh.len into sh.pre (int32; flags a total >= 2^31 or != tokens).
__device__ inline void offsets(int32_t n, int64_t tokens, MetaShared& sh) {
  const int t = threadIdx.x;
  int64_t mine[META_PER_THREAD], excl[META_PER_THREAD];
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int i = t * META_PER_THREAD + e;
    mine[e] = i < n ? sh.len[i] : 0;
  }
  const int64_t total = block_prefix(mine, excl, sh.scan, &sh.total);
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int i = t * META_PER_THREAD + e;
    if (i < n) sh.pre[i] = int32_t(excl[e]);
  }
  if (t == 0) {
    sh.pre[n] = int32_t(total);
    if (total != tokens || total >= (int64_t(1) << 31)) atomicOr(&sh.bad, 1);
  }
  __syncthreads();
}

// Validates and derives the packing metadata of one call into the workspace.
__global__ void __launch_bounds__(META_THREADS)
meta_kernel(const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
            const int32_t* __restrict__ frames, const int32_t* __restrict__ cu_in, int32_t n, int64_t tokens,
            char* __restrict__ ws,
            int64_t off_len, int64_t off_cu, int64_t off_pcu, int64_t off_tiles,
            int64_t tile_capacity) {
  __shared__ MetaShared sh;
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  int32_t* len = reinterpret_cast<int32_t*>(ws + off_len);
  int32_t* cu = reinterpret_cast<int32_t*>(ws + off_cu);
  int32_t* pcu = reinterpret_cast<int32_t*>(ws + off_pcu);
  int2* tiles = reinterpret_cast<int2*>(ws + off_tiles);
  const int t = threadIdx.x;
  if (n <= 64) {
    // Up to 64 samples: one wave, one lane per sample, wave-level scans.
    if (t < 64) meta_small(grid_hw, text_len, frames, cu_in, n, tokens, hdr, len, cu, pcu, tiles);
    return;
  }

  load_lengths(grid_hw, text_len, frames, n, sh);
  offsets(n, tokens, sh);
  // The caller's offsets must be exactly these prefix sums.
  for (int i = t; i <= n; i += META_THREADS) {
    if (cu_in[i] != sh.pre[i]) atomicOr(&sh.bad, 1);
  }
  __syncthreads();
  if (sh.bad != 0) {
    if (t == 0) {
      hdr->flag = FLAG_METADATA;
      hdr->n_tiles = 0;
      hdr->padded_total = 0;
      hdr->n_seg = n;
    }
    return;
  }
  for (int i = t; i < n; i += META_THREADS) {
    len[i] = sh.len[i];
    cu[i] = sh.pre[i];
  }
  if (t == 0) cu[n] = sh.pre[n];

  // Longest-first order of samples (rank by decreasing length, ties by index).
  for (int i = t; i < n; i += META_THREADS) {
    const int32_t li = sh.len[i];
    int32_t rank = 0;
    for (int j = 0; j < n; ++j) {
      const int32_t lj = sh.len[j];
      rank += (lj > li) || (lj == li && j < i);
    }
    sh.order[rank] = i;
  }
  __syncthreads();

  int64_t mine[META_PER_THREAD], excl[META_PER_THREAD];
  // Padded offsets, sample order: every sample rounded up to KTILE rows.
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int i = t * META_PER_THREAD + e;
    mine[e] = i < n ? round_up(sh.len[i], KTILE) : 0;
  }
  const int64_t padded_total = block_prefix(mine, excl, sh.scan, &sh.total);
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int i = t * META_PER_THREAD + e;
    if (i < n) pcu[i] = int32_t(excl[e]);
  }
  if (t == 0) pcu[n] = int32_t(padded_total);

  // Tile offsets in longest-first order: the tiles of order[r] start at pre[r].
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int r = t * META_PER_THREAD + e;
    mine[e] = r < n ? ceil_div(sh.len[sh.order[r]], QTILE) : 0;
  }
  const int64_t total_tiles = block_prefix(mine, excl, sh.scan, &sh.total);
  for (int e = 0; e < META_PER_THREAD; ++e) {
    const int r = t * META_PER_THREAD + e;
    if (r < n) sh.pre[r] = int32_t(excl[e]);
  }
  if (t == 0) sh.pre[n] = int32_t(total_tiles);
  __syncthreads();
  // total_tiles <= ceil(T / QTILE) + n = tile_capacity by construction.
  for (int64_t x = t; x < total_tiles && x < tile_capacity; x += META_THREADS) {
    int32_t lo = 0, hi = n;  // largest r with pre[r] <= x
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (sh.pre[mid] <= x) lo = mid; else hi = mid;
    }
    tiles[x] = make_int2(sh.order[lo], int32_t((x - sh.pre[lo]) * QTILE));
  }
  if (t == 0) {
    hdr->flag = FLAG_OK;
    hdr->n_tiles = int32_t(total_tiles);
    hdr->padded_total = int32_t(padded_total);
    hdr->n_seg = n;
  }
}

// Offsets only (for mf_build_metadata): cu_out = prefix sums; ORs
// FLAG_METADATA into *status when a sample is out of range or the packed
// length differs from `tokens`.
__global__ void __launch_bounds__(META_THREADS)
offsets_kernel(const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
               const int32_t* __restrict__ frames, int32_t n, int64_t tokens, int32_t* __restrict__ cu_out,
               int32_t* __restrict__ status) {
  __shared__ MetaShared sh;
  load_lengths(grid_hw, text_len, frames, n, sh);
  offsets(n, tokens, sh);
  for (int i = threadIdx.x; i <= n; i += META_THREADS) cu_out[i] = sh.pre[i];
  if (threadIdx.x == 0 && sh.bad) atomicOr(status, FLAG_METADATA);
}

// Per-token position and sample id, for tokens below both the capacity and
// cu[n]. THREE: (row, col, frame) per token, else (row, col).
template <bool THREE>
__global__ void __launch_bounds__(256)
positions_kernel(const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
                 const int32_t* __restrict__ cu, int32_t n, int64_t tokens,
                 int32_t* __restrict__ pos, int32_t* __restrict__ seg_id) {
  const int64_t x = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (x >= tokens || x >= cu[n]) return;
  const int32_t i = upper_segment(cu, n, x);
  int32_t r, c, f;
  token_position3(int32_t(x - cu[i]), text_len[i], max(grid_hw[2 * i], 1), max(grid_hw[2 * i + 1], 1), r, c, f);
  if (THREE) {
    pos[3 * x] = r;
    pos[3 * x + 1] = c;
    pos[3 * x + 2] = f;
  } else {
    pos[2 * x] = r;
    pos[2 * x + 1] = c;
  }
  seg_id[x] = i;
}

hipError_t launch_meta(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                       const int32_t* cu_in, int32_t n, int64_t tokens, char* ws, const WsLayout& l,
                       hipStream_t s) {
  hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(META_THREADS), 0, s, grid_hw, text_len, frames, cu_in, n,
                     tokens, ws, l.off_len, l.off_cu, l.off_pcu, l.off_tiles, l.n_tiles);
  return hipGetLastError();
}

hipError_t launch_build_metadata(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                 int32_t n, int64_t tokens, int32_t* cu_out, int32_t* pos, int32_t* seg_id,
                                 int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(META_THREADS), 0, s, grid_hw, text_len, frames, n,
                     tokens, cu_out, status);
  const int64_t blocks = ceil_div(tokens, 256);
  if (frames) {
    hipLaunchKernelGGL(positions_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, s, grid_hw, text_len,
                       cu_out, n, tokens, pos, seg_id);
  } else {
    hipLaunchKernelGGL(positions_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, s, grid_hw, text_len,
                       cu_out, n, tokens, pos, seg_id);
  }
  return hipGetLastError();
}

}  // namespace mf
