// Packing metadata of a batch of at most 64 samples derived by one wave
// (lane i = sample i), with no LDS and no workgroup barrier: shared by the
// metadata kernel and the attention prologue, which derives it itself for
// such batches instead of waiting for a separate metadata launch.
// Source: Mage-Flow tech report, NR-MMDiT section (samples packed back to
// back, attention kept inside each by per-sample cumulative offsets; the
// editing paragraph puts the prompt before the latents).
#pragma once

#include "mf_common.h"

namespace mf {

constexpr int32_t MAX_TEXT_LEN = 1 << 30;

// L_i of sample i and its range checks: 1 <= h, w <= ROPE_PMAX,
// 0 <= text_len <= 2^30, 1 <= frames <= ROPE_PMAX (frames == nullptr: one image).
__device__ inline int32_t sample_length(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                        int i, bool& ok) {
  const int32_t h = grid_hw[2 * i], w = grid_hw[2 * i + 1], tl = text_len[i];
  const int32_t f = frames ? frames[i] : 1;
  ok = h >= 1 && w >= 1 && h <= ROPE_PMAX && w <= ROPE_PMAX && tl >= 0 && tl <= MAX_TEXT_LEN && f >= 1 &&
       f <= ROPE_PMAX;
  return ok ? tl + f * h * w : 1;  // f h w <= 2^27: no overflow
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ inline int64_t wave_inclusive_scan(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// The same derivation as meta_kernel for n <= 64, by the first wave alone:
// lane i owns sample i. No LDS and no workgroup barriers.
__device__ inline void meta_small(const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len,
                                  const int32_t* __restrict__ frames, const int32_t* __restrict__ cu_in,
                                  int32_t n, int64_t tokens,
                                  WsHeader* hdr, int32_t* len, int32_t* cu, int32_t* pcu, int2* tiles) {
  const int i = threadIdx.x;
  const bool mine = i < n;
  int32_t L = 0;
  bool ok = true;
  if (mine) L = sample_length(grid_hw, text_len, frames, i, ok);
  const int64_t incl = wave_inclusive_scan(L);
  const int64_t total = __shfl(incl, 63);
  const int64_t excl = incl - L;
  if (mine && int64_t(cu_in[i]) != excl) ok = false;
  if (i == 0 && (int64_t(cu_in[n]) != total || total != tokens || total >= (int64_t(1) << 31))) ok = false;
  if (__any(!ok)) {
    if (i == 0) {
      hdr->flag = FLAG_METADATA;
      hdr->n_tiles = 0;
      hdr->padded_total = 0;
      hdr->n_seg = n;
    }
    return;
  }
  const int32_t padded = int32_t(round_up(L, KTILE));
  const int64_t pincl = wave_inclusive_scan(padded);
  // Longest-first rank, ties by index; tiles of sample i start after those of
  // every sample ranked before it.
  const int32_t ct = mine ? int32_t(ceil_div(L, QTILE)) : 0;
  int32_t rank = 0, toff = 0;
  for (int j = 0; j < n; ++j) {
    const int32_t lj = __shfl(L, j);
    const int32_t cj = __shfl(ct, j);
    const bool before = (lj > L) || (lj == L && j < i);
    rank += before;
    toff += before ? cj : 0;
  }
  (void)rank;
  // Shuffles run with the whole wave active, before any lane-dependent branch.
  const int32_t total_tiles = int32_t(__shfl(wave_inclusive_scan(ct), 63));
  const int32_t padded_total = int32_t(__shfl(pincl, 63));
  if (mine) {
    len[i] = L;
    cu[i] = int32_t(excl);
    pcu[i] = int32_t(pincl - padded);
    for (int32_t x = 0; x < ct; ++x) tiles[toff + x] = make_int2(i, x * QTILE);
  }
  if (i == 0) {
    cu[n] = int32_t(total);
    pcu[n] = padded_total;
    hdr->flag = FLAG_OK;
    hdr->n_tiles = total_tiles;
    hdr->padded_total = padded_total;
    hdr->n_seg = n;
  }
}

}  // namespace mf
