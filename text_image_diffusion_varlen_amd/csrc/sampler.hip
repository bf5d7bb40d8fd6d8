// Guided rectified-flow Euler step over a packed classifier-free-guidance batch.
//
// Sources: Mage-Flow tech report, NR-MMDiT section (conditional and
// unconditional branches packed into one forward pass); mageflow.net
// architecture page, section 3 (straight rectified-flow paths, Euler steps).
// Per image b with conditional sample cs and unconditional sample us:
//   z_b[p] <- z_b[p] + dt * (v_u[p] + s * (v_c[p] - v_u[p]))
// where v_c[p] / v_u[p] is the predicted velocity of image token p of sample
// cs / us (token cu[cs] + text_len[cs] + p of the packed batch). Without an
// unconditional sample (us < 0) the step uses v_c. fp32 arithmetic; z is fp32.
//
// One launch. Every workgroup first checks all image -> sample maps and builds
// the image table (first token in z, first velocity row of each branch) in
// LDS (while the first z loads are in flight); all workgroups reach the same
// verdict from the same inputs, so either every workgroup writes or none does.
// Then each thread streams 16-byte chunks (8 channels) of z in a grid-stride
// loop, CFG_UNROLL chunks in flight at a time. HBM-bound: per image token and
// channel it reads z, v_c, v_u and writes z.
#include <algorithm>

#include "mf_common.h"

namespace mf {

#ifndef MF_CFG_UNROLL
#define MF_CFG_UNROLL 1
#endif
#ifndef MF_CFG_MAX_BLOCKS
#define MF_CFG_MAX_BLOCKS 1024
#endif
constexpr int CFG_THREADS = 256;
constexpr int CFG_UNROLL = MF_CFG_UNROLL;  // chunks in flight per thread
constexpr int CFG_MAX_BLOCKS = MF_CFG_MAX_BLOCKS;

// A sample (cu range [a, b), grid h x w, prompt t) can serve image tokens when
// its range matches its grid and prompt and stays inside the packed batch.
__device__ inline bool cfg_sample_ok(int32_t a, int32_t b, int32_t h, int32_t w, int32_t t, int64_t total_tokens) {
  return h >= 1 && w >= 1 && h <= ROPE_PMAX && w <= ROPE_PMAX && t >= 0 && a >= 0 && b <= total_tokens &&
         int64_t(b) - a == int64_t(t) + int64_t(h) * w;
}

__device__ inline void load8(const uint16_t* p, float (&o)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void load8(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Dynamic LDS: zoff[n_img + 1] (first token of image b in z; zoff[n_img] = all
// image tokens), crow[n_img], urow[n_img] (first velocity row of image b's
// conditional / unconditional branch).
template <typename T>
__global__ void __launch_bounds__(CFG_THREADS)
cfg_euler_kernel(float* __restrict__ z, const T* __restrict__ v, const int32_t* __restrict__ cu,
                 const int32_t* __restrict__ grid_hw, const int32_t* __restrict__ text_len, int32_t n_seg,
                 int64_t total_tokens, const int32_t* __restrict__ cond_seg,
                 const int32_t* __restrict__ uncond_seg, int32_t n_img, int32_t image_tokens,
                 int32_t channels, float guidance, float dt, int32_t* __restrict__ status) {
  extern __shared__ int32_t tab[];
  int32_t* zoff = tab;
  int32_t* crow = tab + n_img + 1;
  int32_t* urow = crow + n_img;
  __shared__ int32_t wtot[CFG_THREADS / 64];
  __shared__ int32_t wbad[CFG_THREADS / 64];
  const int t = threadIdx.x;

  // Chunk i is channels [8 (i % groups), +8) of z token i / groups.
  const uint32_t groups = uint32_t(channels) >> 3;
  const uint32_t work = uint32_t(image_tokens) * groups;  // < 2^31, checked on the host
  const uint32_t stride = gridDim.x * CFG_THREADS;
  uint32_t base = blockIdx.x * CFG_THREADS + t;
  float zz[CFG_UNROLL][8];

  // Thread t checks and sizes the contiguous run of images [b0, b1). Every map
  // entry is loaded in one round (indices clamped into range, checks applied
  // afterwards) so the table costs two dependent loads, not one per check.
  const int per = (n_img + CFG_THREADS - 1) / CFG_THREADS;
  const int b0 = min(t * per, n_img), b1 = min(b0 + per, n_img);
  int32_t local = 0;
  bool good = true;
  for (int b = b0; b < b1; ++b) {
    const int32_t cs = cond_seg[b], us = uncond_seg[b];
    const int32_t c = min(max(cs, 0), n_seg - 1), u = min(max(us, 0), n_seg - 1);
    const int32_t ca = cu[c], cb = cu[c + 1], h = grid_hw[2 * c], w = grid_hw[2 * c + 1], ct = text_len[c];
    const int32_t ua = cu[u], ub = cu[u + 1], uh = grid_hw[2 * u], uw = grid_hw[2 * u + 1], ut = text_len[u];
    const bool ok_c = cs >= 0 && cs < n_seg && cfg_sample_ok(ca, cb, h, w, ct, total_tokens);
    const bool ok_u = us == -1 || (us >= 0 && us < n_seg && cfg_sample_ok(ua, ub, uh, uw, ut, total_tokens) &&
                                   uh == h && uw == w);
    good = good && ok_c && ok_u;
    const int32_t hw = ok_c ? h * w : 0;  // <= 512 x 512
    crow[b] = ca + ct;
    urow[b] = us >= 0 ? ua + ut : ca + ct;
    zoff[b] = hw;  // image size for now; replaced by its offset below
    local += hw;   // <= 4096 images of <= 512 x 512 tokens: fits int32
  }
  // The z loads of the first pass depend on nothing but the chunk index: they
  // are issued after this thread's map loads (so that those, which the table
  // waits for, are not queued behind them) and before the table is built,
  // whose latency they overlap.
#pragma unroll
  for (int u = 0; u < CFG_UNROLL; ++u) {
    const uint32_t i = base + u * stride;
    if (i < work) {
      const uint32_t tk = i / groups;
      load8(z + int64_t(tk) * channels + (i - tk * groups) * 8, zz[u]);
    }
  }
  // Block-wide exclusive scan of `local`: shuffles inside each wave, then the
  // four wave totals through LDS.
  const int lane = t & 63, wave = t >> 6;
  int32_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const bool wave_bad = __any(!good);
  if (lane == 63) {
    wtot[wave] = incl;
    wbad[wave] = wave_bad;
  }
  __syncthreads();
  int32_t before = 0, total = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < CFG_THREADS / 64; ++i) {
    before += i < wave ? wtot[i] : 0;
    total += wtot[i];
    bad = bad || wbad[i];
  }
  bad = bad || total != image_tokens;
  if (bad) {
    if (blockIdx.x == 0 && t == 0) atomicOr(status, FLAG_METADATA);
    return;
  }
  int32_t run = before + incl - local;
  for (int b = b0; b < b1; ++b) {
    const int32_t hw = zoff[b];
    zoff[b] = run;
    run += hw;
  }
  if (t == 0) zoff[n_img] = total;
  __syncthreads();

  for (bool first = true; base < work; base += CFG_UNROLL * stride, first = false) {
    float vc[CFG_UNROLL][8], vu[CFG_UNROLL][8];
    float* zp[CFG_UNROLL];
#pragma unroll
    for (int u = 0; u < CFG_UNROLL; ++u) {
      const uint32_t i = base + u * stride;
      zp[u] = nullptr;
      if (i >= work) continue;
      const uint32_t tk = i / groups;
      const uint32_t c0 = (i - tk * groups) * 8;
      // image holding token tk: largest b with zoff[b] <= tk
      int32_t lo = 0, hi = n_img;
      while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (uint32_t(zoff[mid]) <= tk) lo = mid; else hi = mid;
      }
      const int64_t p = int64_t(tk) - zoff[lo];
      load8(v + (crow[lo] + p) * channels + c0, vc[u]);
      load8(v + (urow[lo] + p) * channels + c0, vu[u]);
      zp[u] = z + int64_t(tk) * channels + c0;
      if (!first) load8(zp[u], zz[u]);
    }
#pragma unroll
    for (int u = 0; u < CFG_UNROLL; ++u) {
      if (!zp[u]) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) zz[u][e] += dt * (vu[u][e] + guidance * (vc[u][e] - vu[u][e]));
      float4* o = reinterpret_cast<float4*>(zp[u]);
      o[0] = make_float4(zz[u][0], zz[u][1], zz[u][2], zz[u][3]);
      o[1] = make_float4(zz[u][4], zz[u][5], zz[u][6], zz[u][7]);
    }
  }
}

size_t cfg_lds_bytes(int32_t n_img) { return size_t(3 * n_img + 1) * 4; }

hipError_t launch_cfg_euler(float* z, const void* v, const int32_t* cu, const int32_t* grid_hw,
                            const int32_t* text_len, int32_t n_seg, int64_t total_tokens,
                            const int32_t* cond_seg, const int32_t* uncond_seg, int32_t n_img,
                            int64_t image_tokens, int32_t channels, bool bf16, float guidance, float dt,
                            int32_t* status, hipStream_t s) {
  const size_t lds = cfg_lds_bytes(n_img);
  const int64_t chunks = image_tokens * (channels / 8);
  const int32_t blocks = int32_t(std::min<int64_t>(ceil_div(chunks, CFG_THREADS * CFG_UNROLL), CFG_MAX_BLOCKS));
  const int32_t it = int32_t(image_tokens);
  if (bf16) {
    hipLaunchKernelGGL(cfg_euler_kernel<uint16_t>, dim3(blocks), dim3(CFG_THREADS), lds, s, z,
                       static_cast<const uint16_t*>(v), cu, grid_hw, text_len, n_seg, total_tokens, cond_seg,
                       uncond_seg, n_img, it, channels, guidance, dt, status);
  } else {
    hipLaunchKernelGGL(cfg_euler_kernel<float>, dim3(blocks), dim3(CFG_THREADS), lds, s, z,
                       static_cast<const float*>(v), cu, grid_hw, text_len, n_seg, total_tokens, cond_seg,
                       uncond_seg, n_img, it, channels, guidance, dt, status);
  }
  return hipGetLastError();
}

}  // namespace mf
