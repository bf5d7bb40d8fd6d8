// Joint-layout pack and unpack of the two modality streams.
//
// Source: Mage-Flow tech report, NR-MMDiT section. Text and visual tokens go
// through modality-specific layers and are concatenated, sample by sample,
// for the joint attention; prompts and images are each packed without
// padding. So the attention's joint rows are, for every sample i, its T_i
// prompt rows followed by its image rows (f_i h_i w_i of them: one grid, or
// the images of an edit one after another), while the projections produce
// two packed streams: the text stream (all prompts back to back) and the
// image stream (all images back to back).
//
// pack:   joint[cu[i] + u] = u < T_i ? text[tcu[i] + u] : image[icu[i] + u - T_i]
// unpack: the same map with source and destination exchanged,
// with tcu[i] = sum_{j<i} T_j and icu[i] = cu[i] - tcu[i].
//
// Pure data movement, HBM-bound: every row is read once and written once.
// One launch moves up to MAX_TENSORS tensors (q, k, v together). Each
// workgroup first loads the whole batch's metadata into LDS, checks it
// (cu_seqlens equal to the prefix sums of T_i + f_i h_i w_i, sides in range,
// the two streams' lengths) and forms tcu with a workgroup scan; if any check
// fails it writes nothing and flags the status word. Then it copies rows in a
// grid-stride loop, one wave per row: the wave finds the row's sample by a
// binary search in the LDS copy of cu_seqlens and moves the row as 16-byte
// chunks, every load of the row issued before its stores.
#include "mf_common.h"

namespace mf {

constexpr int PACK_THREADS = 256;
constexpr int PACK_WAVES = PACK_THREADS / 64;
constexpr int PACK_MAX_TENSORS = 4;
constexpr int PACK_PER_THREAD = MAX_SEGMENTS / PACK_THREADS;  // 16
#ifndef MF_PACK_ROWS
#define MF_PACK_ROWS 2
#endif
#ifndef MF_PACK_WG_PER_CU
#define MF_PACK_WG_PER_CU 4
#endif
constexpr int PACK_CHUNKS = 8 * MF_PACK_ROWS;  // 16-byte chunks per lane in flight
constexpr int PACK_ROWS = MF_PACK_ROWS;        // rows per wave and step when they fit in PACK_CHUNKS

struct PackArgs {
  const char* src[PACK_MAX_TENSORS][2];  // pack: (text, image) stream of each tensor; unpack: (joint, -)
  char* dst[PACK_MAX_TENSORS][2];        // pack: (joint, -); unpack: (text, image)
  const int32_t* cu;
  const int32_t* grid_hw;
  const int32_t* text_len;
  const int32_t* frames;  // may be null (one image per sample)
  int32_t* status;
  int32_t n_seg;
  int32_t n_tensors;
  int64_t tokens;       // joint rows
  int64_t text_tokens;  // rows of the text stream
  int32_t row_chunks;   // 16-byte chunks per row
};

// LDS image of the metadata, sized to the batch (dynamic shared memory):
// part[PACK_THREADS], bad, cu[n + 1], tcu[n + 1], text[n].
__host__ __device__ inline size_t pack_lds_bytes(int32_t n) { return size_t(PACK_THREADS + 1 + 3 * n + 2) * 4; }

// Keeps the compiler from sinking the loads above it down to their stores
// (which would leave one load in flight per wave).
__device__ inline void loads_before_stores() { __builtin_amdgcn_sched_barrier(0); }

typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk, held in 4 VGPRs

// Copies one row of c16 16-byte chunks in pieces of 64 * PACK_CHUNKS chunks;
// in a piece lane l moves chunks l, l + 64, ..., all loads before the stores.
// Loads are unconditional (a lane past the row's end re-reads its last chunk)
// so that they issue back to back; only the stores are masked.
__device__ inline void copy_row(const chunk_t* __restrict__ s, chunk_t* __restrict__ d, int c16, int lane) {
  for (int base = 0; base < c16; base += 64 * PACK_CHUNKS) {
    chunk_t v[PACK_CHUNKS];
#pragma unroll
    for (int i = 0; i < PACK_CHUNKS; ++i) v[i] = s[min(base + lane + 64 * i, c16 - 1)];
    loads_before_stores();
#pragma unroll
    for (int i = 0; i < PACK_CHUNKS; ++i)
      if (base + lane + 64 * i < c16) d[base + lane + 64 * i] = v[i];
  }
}

template <bool UNPACK>
__global__ void __launch_bounds__(PACK_THREADS) pack_kernel(PackArgs a) {
  extern __shared__ int32_t lds[];
  const int t = threadIdx.x;
  const int32_t n = a.n_seg;
  struct {
    int32_t* part;
    int32_t& bad;
    int32_t* cu;
    int32_t* tcu;
    int32_t* text;
  } sh{lds, lds[PACK_THREADS], lds + PACK_THREADS + 1, lds + PACK_THREADS + 1 + (n + 1),
       lds + PACK_THREADS + 1 + 2 * (n + 1)};
  if (t == 0) sh.bad = 0;
  __syncthreads();
  // Metadata: lengths checked against cu_seqlens; prompt lengths scanned.
  int32_t mine = 0;
  for (int e = 0; e < PACK_PER_THREAD; ++e) {
    const int i = t * PACK_PER_THREAD + e;
    if (i >= n) break;
    const int32_t h = a.grid_hw[2 * i], w = a.grid_hw[2 * i + 1], tl = a.text_len[i];
    const int32_t f = a.frames ? a.frames[i] : 1;
    const int32_t c0 = a.cu[i], c1 = a.cu[i + 1];
    const bool ok = h >= 1 && w >= 1 && h <= ROPE_PMAX && w <= ROPE_PMAX && f >= 1 && f <= ROPE_PMAX && tl >= 0 &&
                    int64_t(c1) - c0 == int64_t(tl) + int64_t(f) * h * w;
    if (!ok) atomicOr(&sh.bad, 1);
    sh.cu[i] = c0;
    sh.text[i] = tl;
    mine += ok ? tl : 0;
  }
  if (t == 0) {
    sh.cu[n] = a.cu[n];
    if (a.cu[0] != 0 || int64_t(a.cu[n]) != a.tokens) atomicOr(&sh.bad, 1);
  }
  // Exclusive scan of the per-thread prompt totals (Hillis-Steele in LDS).
  sh.part[t] = mine;
  __syncthreads();
  for (int off = 1; off < PACK_THREADS; off <<= 1) {
    const int32_t y = t >= off ? sh.part[t - off] : 0;
    __syncthreads();
    sh.part[t] += y;
    __syncthreads();
  }
  int32_t run = sh.part[t] - mine;
  for (int e = 0; e < PACK_PER_THREAD; ++e) {
    const int i = t * PACK_PER_THREAD + e;
    if (i >= n) break;
    sh.tcu[i] = run;
    run += sh.text[i];
  }
  if (t == PACK_THREADS - 1) {
    sh.tcu[n] = sh.part[t];
    if (int64_t(sh.part[t]) != a.text_tokens) atomicOr(&sh.bad, 1);
  }
  __syncthreads();
  if (sh.bad) {
    if (blockIdx.x == 0 && t == 0) atomicOr(a.status, FLAG_METADATA);
    return;
  }

  const int wave = t >> 6, lane = t & 63;
  const int64_t rows = a.tokens * a.n_tensors;
  const int c16 = a.row_chunks;
  const int64_t row_bytes = int64_t(c16) * 16;
  // Source and destination of joint row x (tensor-major over all tensors).
  auto row_ptrs = [&](int64_t x, const chunk_t*& src, chunk_t*& dst) {
    const int tensor = int(x / a.tokens);
    const int32_t r = int32_t(x - int64_t(tensor) * a.tokens);
    int32_t lo = 0, hi = n;  // sample: largest i with cu[i] <= r
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (sh.cu[mid] <= r) lo = mid; else hi = mid;
    }
    const int32_t u = r - sh.cu[lo];
    const bool is_text = u < sh.text[lo];
    const int64_t srow = is_text ? int64_t(sh.tcu[lo]) + u : int64_t(sh.cu[lo]) - sh.tcu[lo] + (u - sh.text[lo]);
    if constexpr (UNPACK) {
      src = reinterpret_cast<const chunk_t*>(a.src[tensor][0] + int64_t(r) * row_bytes);
      dst = reinterpret_cast<chunk_t*>(a.dst[tensor][is_text ? 0 : 1] + srow * row_bytes);
    } else {
      src = reinterpret_cast<const chunk_t*>(a.src[tensor][is_text ? 0 : 1] + srow * row_bytes);
      dst = reinterpret_cast<chunk_t*>(a.dst[tensor][0] + int64_t(r) * row_bytes);
    }
  };
  // Each wave moves PACK_ROWS consecutive rows per step (their loads all in
  // flight together when a row is at most 64 * PACK_CHUNKS / PACK_ROWS chunks).
  const int64_t step = int64_t(gridDim.x) * PACK_WAVES * PACK_ROWS;
  for (int64_t x0 = (int64_t(blockIdx.x) * PACK_WAVES + wave) * PACK_ROWS; x0 < rows; x0 += step) {
    if (c16 * PACK_ROWS <= 64 * PACK_CHUNKS) {
      constexpr int PER_ROW = PACK_CHUNKS / PACK_ROWS;
      const chunk_t* src[PACK_ROWS];
      chunk_t* dst[PACK_ROWS];
      chunk_t v[PACK_ROWS][PER_ROW];
#pragma unroll
      for (int k = 0; k < PACK_ROWS; ++k) {
        // rows past the end re-read the last row (their stores are masked)
        row_ptrs(min(x0 + k, rows - 1), src[k], dst[k]);
#pragma unroll
        for (int i = 0; i < PER_ROW; ++i) v[k][i] = src[k][min(lane + 64 * i, c16 - 1)];
      }
      loads_before_stores();
#pragma unroll
      for (int k = 0; k < PACK_ROWS; ++k) {
#pragma unroll
        for (int i = 0; i < PER_ROW; ++i)
          if (x0 + k < rows && lane + 64 * i < c16) dst[k][lane + 64 * i] = v[k][i];
      }
    } else {
      for (int k = 0; k < PACK_ROWS && x0 + k < rows; ++k) {
        const chunk_t* src;
        chunk_t* dst;
        row_ptrs(x0 + k, src, dst);
        copy_row(src, dst, c16, lane);
      }
    }
  }
}

// pack == true: src[i] = (text_i, image_i), dst[i] = joint_i; else the reverse.
hipError_t launch_pack(bool unpack, int32_t n_tensors, const void* const* src0, const void* const* src1,
                       void* const* dst0, void* const* dst1, const int32_t* cu, const int32_t* grid_hw,
                       const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t tokens,
                       int64_t text_tokens, int64_t row_bytes, int32_t ncu, int32_t* status, hipStream_t s) {
  PackArgs a{};
  for (int i = 0; i < n_tensors; ++i) {
    a.src[i][0] = static_cast<const char*>(src0[i]);
    a.src[i][1] = src1 ? static_cast<const char*>(src1[i]) : nullptr;
    a.dst[i][0] = static_cast<char*>(dst0[i]);
    a.dst[i][1] = dst1 ? static_cast<char*>(dst1[i]) : nullptr;
  }
  a.cu = cu;
  a.grid_hw = grid_hw;
  a.text_len = text_len;
  a.frames = frames;
  a.status = status;
  a.n_seg = n_seg;
  a.n_tensors = n_tensors;
  a.tokens = tokens;
  a.text_tokens = text_tokens;
  a.row_chunks = int32_t(row_bytes / 16);
  // Persistent grid: a few workgroups per CU, each checking the metadata once
  // and then streaming rows; no more workgroups than row pairs per wave.
  const int64_t want = ceil_div(tokens * n_tensors, PACK_WAVES * PACK_ROWS);
  const int64_t cap = MF_PACK_WG_PER_CU > 0 ? int64_t(ncu > 0 ? ncu : 256) * MF_PACK_WG_PER_CU : want;
  const dim3 grid(unsigned(want < cap ? want : cap));
  const size_t lds = pack_lds_bytes(n_seg);
  if (unpack) hipLaunchKernelGGL(pack_kernel<true>, grid, dim3(PACK_THREADS), lds, s, a);
  else hipLaunchKernelGGL(pack_kernel<false>, grid, dim3(PACK_THREADS), lds, s, a);
  return hipGetLastError();
}

}  // namespace mf
